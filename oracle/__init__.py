"""CPU oracle of the fused Dr. GRPO loss: binary64, plain loops, slow.

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``rl_post_loss_dr_amd``) never imports it and fails loudly when its own
HIP library is missing.

The arithmetic lives in ``drgrpo_oracle.c`` (compiled with gcc, no HIP); this
module only marshals numpy arrays and composes its steps in the pages' order:
completion mask -> group advantage -> log-softmax + gather -> clipped
surrogate (+ k3 KL) -> token sum / kappa -> gradient rows.  The GRPO
normalisations (group-std advantage, per-response mean) and the token mean are
selected by ``adv_mode`` / ``agg``.  The fused lm_head
variant (logits = hidden @ W^T) is in ``lmhead.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64 = 0, 1, 2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double


def build(verbose: bool = False) -> None:
    """Compile drgrpo_oracle.c with gcc (no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-o", LIB, os.path.join(_HERE, "drgrpo_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run oracle.build()")
        L = ctypes.CDLL(LIB)
        L.oracle_completion_len.argtypes = [_P, _I64, _I64, _I64, _P]
        L.oracle_completion_len.restype = ctypes.c_int
        L.oracle_group_advantage.argtypes = [_P, _I64, _I64, _P]
        L.oracle_group_advantage.restype = ctypes.c_int
        L.oracle_group_advantage_zscore.argtypes = [_P, _I64, _I64, _P]
        L.oracle_group_advantage_zscore.restype = ctypes.c_int
        L.oracle_row_divisor.argtypes = [_P, _I64, ctypes.c_int, _D, _P]
        L.oracle_row_divisor.restype = ctypes.c_int
        L.oracle_nocontrast_groups.argtypes = [_P, _I64, _I64]
        L.oracle_nocontrast_groups.restype = _I64
        L.oracle_row_logprob.argtypes = [_P, ctypes.c_int, _I64, _P, _I64, _P, _P]
        L.oracle_row_logprob.restype = _I64
        L.oracle_token_terms.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _D, _D, _P, _P, _P, _P]
        L.oracle_token_terms.restype = ctypes.c_int
        L.oracle_loss.argtypes = [_P, _P, _I64, _I64]
        L.oracle_loss.restype = _D
        L.oracle_dlogits_rows.argtypes = [_P, ctypes.c_int, _I64, _P, _P, _P, _I64, _P]
        L.oracle_dlogits_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _logits_code(x: np.ndarray, dtype: int | None) -> tuple[np.ndarray, int]:
    """Logits as stored: float32, bfloat16 bits (uint16) or float64."""
    if x.dtype == np.float32:
        return _c(x, np.float32), F32
    if x.dtype == np.uint16:
        return _c(x, np.uint16), BF16
    if x.dtype == np.float64:
        return _c(x, np.float64), F64
    raise TypeError(f"logits dtype {x.dtype}: pass float32, float64 or bf16 bits as uint16")


# ------------------------------------------------------------------------ steps
def completion_len(tokens: np.ndarray, eos_id: int) -> np.ndarray:
    tokens = _c(tokens, np.int64)
    N, C = tokens.shape
    out = np.empty(N, dtype=np.int32)
    if lib().oracle_completion_len(tokens.ctypes.data, N, C, eos_id, out.ctypes.data) != 0:
        raise ValueError("bad arguments")
    return out


def completion_mask(tokens: np.ndarray, eos_id: int) -> np.ndarray:
    L = completion_len(tokens, eos_id)
    return (np.arange(tokens.shape[1])[None, :] < L[:, None]).astype(np.uint8)


ADV_CENTER, ADV_ZSCORE = 0, 1                      # Dr. GRPO, GRPO advantages
AGG_TOKEN_SUM, AGG_SEQ_MEAN, AGG_TOKEN_MEAN = 0, 1, 2  # aggregation divisors


def group_advantage(rewards: np.ndarray, G: int, mode: int = ADV_CENTER) -> np.ndarray:
    rewards = _c(rewards, np.float32)
    out = np.empty_like(rewards)
    fn = lib().oracle_group_advantage if mode == ADV_CENTER else \
        lib().oracle_group_advantage_zscore
    if mode not in (ADV_CENTER, ADV_ZSCORE) or \
            fn(rewards.ctypes.data, rewards.size, G, out.ctypes.data) != 0:
        raise ValueError("bad arguments")
    return out


def row_divisor(lens: np.ndarray, kappa: float, agg: int = AGG_TOKEN_SUM) -> np.ndarray:
    """Per-completion divisor of the token sums (see oracle_row_divisor)."""
    lens = _c(lens, np.int32).reshape(-1)
    out = np.empty(lens.size, dtype=np.float64)
    if lib().oracle_row_divisor(lens.ctypes.data, lens.size, agg, kappa, out.ctypes.data) != 0:
        raise ValueError("bad arguments")
    return out


def nocontrast_groups(rewards: np.ndarray, G: int) -> int:
    rewards = _c(rewards, np.float32)
    n = lib().oracle_nocontrast_groups(rewards.ctypes.data, rewards.size, G)
    if n < 0:
        raise ValueError("bad arguments")
    return int(n)


def row_logprob(logits2d: np.ndarray, tokens_flat: np.ndarray) -> tuple[np.ndarray, np.ndarray, int]:
    """(lse, logp, n_bad_tokens) for each row of a [R, V] logits array."""
    x, code = _logits_code(logits2d, None)
    R, V = x.shape
    tok = _c(tokens_flat, np.int64).reshape(-1)
    assert tok.size == R
    lse = np.empty(R, dtype=np.float64)
    logp = np.empty(R, dtype=np.float64)
    bad = lib().oracle_row_logprob(x.ctypes.data, code, V, tok.ctypes.data, R, lse.ctypes.data,
                                   logp.ctypes.data)
    if bad < 0:
        raise ValueError("bad arguments")
    return lse, logp, int(bad)


def token_terms(logp, logp_old, logp_ref, adv, lens, eps, beta, kappa, agg=AGG_TOKEN_SUM):
    """(lambda, coef, stats[2]) per token of a [N, C] batch."""
    logp = _c(logp, np.float64)
    N, C = logp.shape
    old = _c(logp_old, np.float32)
    ref = None if logp_ref is None else _c(logp_ref, np.float32)
    adv = _c(adv, np.float32)
    lens = _c(lens, np.int32)
    lam = np.empty((N, C), dtype=np.float64)
    coef = np.empty((N, C), dtype=np.float64)
    stats = np.zeros(2, dtype=np.int64)
    div = row_divisor(lens, kappa, agg)
    rc = lib().oracle_token_terms(logp.ctypes.data, old.ctypes.data,
                                  None if ref is None else ref.ctypes.data, adv.ctypes.data,
                                  lens.ctypes.data, N, C, eps, beta, div.ctypes.data,
                                  lam.ctypes.data, coef.ctypes.data, stats.ctypes.data)
    if rc != 0:
        raise ValueError("bad arguments")
    return lam, coef, stats


def loss_sum(lam: np.ndarray, kappa: float, lens=None, agg: int = AGG_TOKEN_SUM) -> float:
    """L from the per-token terms lam [N, C] (a flat array is one row per
    entry); lens is needed for the per-response and token-mean divisors."""
    lam = _c(lam, np.float64)
    lam2 = lam.reshape(lam.shape[0], -1) if lam.ndim > 1 else lam.reshape(-1, 1)
    N, C = lam2.shape
    if lens is None:
        if agg != AGG_TOKEN_SUM:
            raise ValueError("lens is needed for this aggregation")
        lens = np.ones(N, dtype=np.int32)
    div = row_divisor(lens, kappa, agg)
    return float(lib().oracle_loss(lam2.ctypes.data, div.ctypes.data, N, C))


def dlogits_rows(logits2d, tokens_flat, lse, coef) -> np.ndarray:
    x, code = _logits_code(logits2d, None)
    R, V = x.shape
    tok = _c(tokens_flat, np.int64).reshape(-1)
    lse = _c(lse, np.float64).reshape(-1)
    coef = _c(coef, np.float64).reshape(-1)
    out = np.empty((R, V), dtype=np.float64)
    if lib().oracle_dlogits_rows(x.ctypes.data, code, V, tok.ctypes.data, lse.ctypes.data,
                                 coef.ctypes.data, R, out.ctypes.data) != 0:
        raise ValueError("bad arguments")
    return out


# ------------------------------------------------------------------ composition
@dataclass
class Result:
    loss: float                 # L in binary64
    dlogits: np.ndarray | None  # [N*C, V] binary64 (None when not requested)
    len: np.ndarray             # int32 [N]
    adv: np.ndarray             # float32 [N]
    lse: np.ndarray             # float64 [N, C]
    logp: np.ndarray            # float64 [N, C]
    lam: np.ndarray             # float64 [N, C] per-token loss term (0 when inactive)
    coef: np.ndarray            # float64 [N, C]
    nocontrast: int
    truncated: int
    stats: np.ndarray           # int64 [2]: ratio outside clip range, clip-cut tokens
    bad_tokens: int

    @property
    def abs_sum(self) -> float:
        """sum of |lambda| over tokens: the scale kappa * L can cancel from."""
        return float(np.abs(self.lam).sum())


def loss_fwd_bwd(logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta, kappa,
                 want_dlogits: bool = True, adv_mode: int = ADV_CENTER,
                 agg: int = AGG_TOKEN_SUM) -> Result:
    """Whole oracle pass for a batch small enough to hold [N*C, V] in memory.

    logits: [N*C, V] (or [N, C, V]) float32 / float64 / bf16 bits as uint16.
    """
    tokens = _c(tokens, np.int64)
    N, C = tokens.shape
    x = logits.reshape(N * C, -1)
    lens = completion_len(tokens, eos_id)
    adv = group_advantage(rewards, G, adv_mode)
    mask = np.arange(C)[None, :] < lens[:, None]
    lse, logp, _ = row_logprob(x, tokens.reshape(-1))
    bad = int(((tokens < 0) | (tokens >= x.shape[1]))[mask].sum())
    lse = lse.reshape(N, C)
    logp = logp.reshape(N, C)
    lam, coef, stats = token_terms(logp, logp_old, logp_ref, adv, lens, eps, beta, kappa, agg)
    L = loss_sum(lam, kappa, lens, agg)
    if bad:
        L = float("nan")
    D = dlogits_rows(x, tokens.reshape(-1), lse.reshape(-1), coef.reshape(-1)) \
        if want_dlogits else None
    return Result(loss=L, dlogits=D, len=lens, adv=adv, lse=lse, logp=logp, lam=lam, coef=coef,
                  nocontrast=nocontrast_groups(rewards, G),
                  truncated=int((~(tokens == eos_id).any(axis=1)).sum()), stats=stats,
                  bad_tokens=bad)
