"""CPU oracle of the fused lm_head variant (binary64).

TEST INFRASTRUCTURE (see the package docstring).  The logits are the
definition hidden . W^T, formed with numpy's binary64 matrix product (a
library routine) for one block of whole token rows at a time; every later
step is the raw-logits oracle of ``drgrpo_oracle.c``; the two weight
gradients are the chain rule through that product, again plain binary64
matrix products:  dL/dhidden = dlogits . W  and  dL/dW = dlogits^T . hidden.
"""
from __future__ import annotations

import numpy as np

from . import completion_len, dlogits_rows, group_advantage, loss_sum, row_logprob, token_terms


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def token_rows(hidden64, W64, tokens_flat, rows, block=256):
    """(lse, logp) of the given token rows, computing full logit rows in blocks."""
    rows = np.asarray(rows, dtype=np.int64)
    lse = np.empty(rows.size)
    logp = np.empty(rows.size)
    for b0 in range(0, rows.size, block):
        r = rows[b0:b0 + block]
        logits = hidden64[r] @ W64.T
        l, p, _ = row_logprob(logits, tokens_flat[r])
        lse[b0:b0 + block] = l
        logp[b0:b0 + block] = p
    return lse, logp


def loss_and_terms(hidden64, W64, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta,
                   kappa, adv_mode=0, agg=0):
    """Loss over every token and the per-token pieces the gradients need."""
    N, C = tokens.shape
    lens = completion_len(tokens, eos_id)
    adv = group_advantage(rewards, G, adv_mode)
    mask = np.arange(C)[None, :] < lens[:, None]
    active = mask & ((adv[:, None] != 0) | (beta != 0))
    rows = np.flatnonzero(active.reshape(-1))
    lse = np.zeros(N * C)
    logp = np.zeros(N * C)
    if rows.size:
        l, p = token_rows(hidden64, W64, tokens.reshape(-1), rows)
        lse[rows] = l
        logp[rows] = p
    lam, coef, stats = token_terms(logp.reshape(N, C), logp_old, logp_ref, adv, lens, eps, beta,
                                   kappa, agg)
    return dict(loss=loss_sum(lam, kappa, lens, agg), lse=lse, logp=logp.reshape(N, C), lam=lam,
                coef=coef.reshape(-1), active_rows=rows, len=lens, adv=adv, stats=stats)


def dlogits_token_rows(hidden64, W64, tokens_flat, terms, rows):
    """dlogits [len(rows), V] of the given token rows (zero rows where the
    token has no gradient): the raw-logits oracle's gradient rows of
    hidden[rows] . W^T."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, W64.shape[0]))
    live = np.flatnonzero(terms["coef"][rows] != 0.0)
    if live.size:
        r = rows[live]
        logits = hidden64[r] @ W64.T
        out[live] = dlogits_rows(logits, tokens_flat[r], terms["lse"][r], terms["coef"][r])
    return out


def dlogits_vocab_cols(hidden64, W64, tokens_flat, terms, vocab_rows):
    """dlogits [active tokens, len(vocab_rows)]: column v of the active tokens'
    gradient rows, dlogits[t, v] = coef_t (exp(logits[t, v] - lse_t) - [y_t = v])."""
    act = terms["active_rows"]
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    Ha = hidden64[act]
    lse = terms["lse"][act]
    coef = terms["coef"][act]
    y = tokens_flat[act]
    cols = Ha @ W64[vocab_rows].T                  # logits[t, v] for the active tokens
    return coef[:, None] * (np.exp(cols - lse[:, None]) - (y[:, None] == vocab_rows[None, :]))


def dhidden_rows(hidden64, W64, tokens_flat, terms, rows):
    """dL/dhidden for the given token rows: (dlogits row) . W."""
    return dlogits_token_rows(hidden64, W64, tokens_flat, terms, rows) @ W64


def dW_rows(hidden64, W64, tokens_flat, terms, vocab_rows):
    """dL/dW for the given vocabulary rows: sum over tokens of dlogits[t, v] * hidden[t]."""
    act = terms["active_rows"]
    out = np.zeros((len(vocab_rows), hidden64.shape[1]))
    if act.size == 0:
        return out
    return dlogits_vocab_cols(hidden64, W64, tokens_flat, terms, vocab_rows).T @ hidden64[act]


def full(hidden_bits, W_bits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta, kappa,
         adv_mode=0, agg=0):
    """Loss, full dhidden [T, H] and dW [V, H] for a case small enough to hold [T, V]."""
    h = bf16_to_f64(hidden_bits)
    W = bf16_to_f64(W_bits)
    terms = loss_and_terms(h, W, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta, kappa,
                           adv_mode, agg)
    logits = h @ W.T
    D = dlogits_rows(logits, tokens.reshape(-1), terms["lse"], terms["coef"])
    terms["dhidden"] = D @ W
    terms["dW"] = D.T @ h
    terms["dlogits"] = D
    return terms
