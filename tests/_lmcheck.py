"""Checks of the fused lm_head's weight gradients against the oracle, built so
that a wrong part of the gradient fails them ("The Quiet Library", section
"A controlled experiment that can answer the question": compare parameter
gradients in the intended precision).

What the GPU computes: every dlogits entry D[t, v] = coef_t (p_tv - [v = y_t])
as s_t E[t, v], with E = exp(x - r_t) from binary32 logits rounded to
bfloat16 and s_t = coef_t exp(r_t - lse_t) in binary32 (r_t a per-token
reference); binary32 products dhidden = s . (E . W) and
dW = E^T . (s . hidden), the scaled hidden rows s_t hidden_t rounded to
bfloat16; bfloat16 results.  Error model of one output element with oracle
value R (binary64), from its terms D x (x = W[v, k] for dhidden,
hidden[t, k] for dW):

  * each term carries n independent roundings to bfloat16 (n = 1 for
    dhidden: E; n = 2 for dW: E and s_t hidden_t), each a relative error
    <= u = 2^-8, zero mean, RMS below u / sqrt(3) (round to nearest even);
  * binary32 logits, binary32 exponentials and binary32 accumulation:
    relative error of order 2^-17 of S = sum |D| |x| (the realised errors of
    all of them are ~1e-5 of S or less);
  * the result is rounded once to bfloat16: relative error <= u, RMS below
    u / sqrt(3).

Three checks follow, each over a named part of the gradient:

  (E) every element:   |got - R| <= u |R| + (n + 1) u S        (worst case:
      n u + (n - 1) u^2 per term, with about u S to spare for the binary32
      steps)
  (F) every row and the part as a whole:
         ||got - R||_F <= 3 sqrt(sum u^2/3 (n Q + R^2)) + ||2^-17 S||_F
      with Q = sum (D x)^2 per element.  The factor 3 covers even one or two
      fully aligned worst-case roundings per element (sqrt(3) sqrt(2) < 3); a
      dropped, zeroed or garbage row is far outside it.
  (S) the part's regression slope <got, R> / <R, R> lies within `slope_tol`
      of 1: the rounding errors are unbiased and average out over the part, a
      systematic error (a scaled or dropped part) does not.

The parts checked at their own scale are the ones a check against the largest
entry of the whole matrix would not see: the vocabulary rows of dW that no
active token sampled (magnitude 1e-2 to 1e-3 of the sampled rows) and the
softmax part of dhidden, coef_t sum_v p_tv W[v] = dhidden_t + coef_t W[y_t]
(about 2% of each row at W ~ N(0, 0.02^2)).
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -8            # bfloat16 unit roundoff
E32 = 2.0 ** -17         # binary32 logits and accumulation, relative to S
FROB_FACTOR = 3.0
SLOPE_TOL = 4e-3         # parts whose reference is the gradient itself
SLOPE_TOL_SOFTMAX = 5e-2  # dhidden's softmax part: ~2% of the row, its rounding noise is larger
SOFTMAX_FROB_REL = 0.5   # ||err|| / ||softmax part|| over the whole part


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 values (ties to even) of finite binary32-range values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _row_frob(err, var, e32):
    """Per-row (F): returns the worst ratio of ||err|| to its bound."""
    lim = FROB_FACTOR * np.sqrt(var.sum(axis=1)) + np.sqrt((e32 * e32).sum(axis=1))
    n = np.sqrt((err * err).sum(axis=1))
    ok = n <= lim
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, n / lim, np.where(n > 0, np.inf, 0.0))
    return ok, ratio


def check_part(name: str, got: np.ndarray, ref: np.ndarray, S: np.ndarray, Q: np.ndarray,
               slope_tol: float | None = SLOPE_TOL, n_round: int = 1) -> dict:
    """(E), (F) per row and whole, (S) for one part whose terms carry n_round
    roundings to bfloat16; raises AssertionError."""
    got = np.asarray(got, dtype=np.float64)
    err = got - ref
    assert np.isfinite(got).all(), f"{name}: non-finite entries"
    bound = U * np.abs(ref) + (n_round + 1) * U * S
    bad = np.abs(err) > bound
    assert not bad.any(), (
        f"{name}: {int(bad.sum())} elements beyond u|R| + {n_round + 1}u S; worst got="
        f"{got[bad][:3]} want={ref[bad][:3]}")
    var = U * U / 3.0 * (n_round * Q + ref * ref)
    e32 = E32 * S
    ok, ratio = _row_frob(err, var, e32)
    assert ok.all(), f"{name}: {int((~ok).sum())} rows beyond the rounding model, worst ratio " \
                     f"{float(ratio.max()):.3g}"
    whole = FROB_FACTOR * np.sqrt(var.sum()) + np.sqrt((e32 * e32).sum())
    assert np.sqrt((err * err).sum()) <= whole, f"{name}: part beyond the rounding model"
    out = {"rows": int(ref.shape[0]), "max_row_ratio": float(ratio.max()) if ratio.size else 0.0}
    rr = float((ref * ref).sum())
    if slope_tol is not None and rr > 0:
        s = float((got * ref).sum()) / rr
        out["slope"] = s
        assert abs(s - 1.0) <= slope_tol, f"{name}: slope {s!r} (tolerance {slope_tol})"
    return out


def check_dhidden(got: np.ndarray, D: np.ndarray, W64: np.ndarray, coef: np.ndarray,
                  y: np.ndarray) -> dict:
    """dhidden rows `got` [n, H] against D [n, V] (the oracle's dlogits rows of
    those tokens) . W; coef [n] and y [n] are the rows' coefficients and
    sampled ids.  Rows with coef = 0 must be exact zeros."""
    ref = D @ W64
    S = np.abs(D) @ np.abs(W64)
    Q = (D * D) @ (W64 * W64)
    res = {"full": check_part("dhidden", got, ref, S, Q)}
    live = coef != 0
    if live.any():
        hard = coef[live, None] * W64[y[live]]
        sm_ref = ref[live] + hard
        sm_got = np.asarray(got, dtype=np.float64)[live] + hard
        err = sm_got - sm_ref
        rel = float(np.sqrt((err * err).sum() / (sm_ref * sm_ref).sum()))
        assert rel <= SOFTMAX_FROB_REL, f"dhidden softmax part: relative error {rel:.3g}"
        s = float((sm_got * sm_ref).sum() / (sm_ref * sm_ref).sum())
        assert abs(s - 1.0) <= SLOPE_TOL_SOFTMAX, f"dhidden softmax part: slope {s!r}"
        res["softmax"] = {"rel": rel, "slope": s}
    return res


def check_dW(got: np.ndarray, Dc: np.ndarray, Ha: np.ndarray, sampled: np.ndarray) -> dict:
    """dW rows `got` [nv, H] for some vocabulary rows against Dc^T . Ha, with
    Dc [T_a, nv] the oracle's dlogits columns of those rows over the active
    tokens and Ha [T_a, H] their hidden rows; `sampled` [nv] marks the rows
    some active token sampled.  The sampled and the other rows are checked as
    separate parts."""
    got = np.asarray(got, dtype=np.float64)
    ref = Dc.T @ Ha
    S = np.abs(Dc).T @ np.abs(Ha)
    Q = (Dc * Dc).T @ (Ha * Ha)
    res = {}
    for label, sel in (("dW sampled rows", sampled), ("dW unsampled rows", ~sampled)):
        if sel.any():
            res[label] = check_part(label, got[sel], ref[sel], S[sel], Q[sel], n_round=2)
    return res


def round_rel(x: np.ndarray, bits: int) -> np.ndarray:
    """x with its significand rounded to `bits` bits (nearest), any exponent:
    the relative rounding of a bfloat16 value (bits = 8) without its range."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def emulate(D: np.ndarray, X: np.ndarray, xscale: np.ndarray | None = None) -> np.ndarray:
    """The GPU's precision path for D . X, emulated on the CPU: each D entry
    carries the relative rounding of a bfloat16 value (8 bits: E rounded,
    then scaled by its token's factor); with xscale [K], row k of X is taken
    as bf16(xscale_k X_k) / xscale_k (the dW product's scaled hidden rows);
    a binary32 product, and the result rounded to bfloat16.  Only the
    checker's own tests use it."""
    Db = round_rel(D, 8).astype(np.float32)
    X = np.asarray(X, dtype=np.float64)
    if xscale is not None:
        sc = np.asarray(xscale, dtype=np.float64)[:, None]
        nz = sc != 0
        X = np.where(nz, bf16_round(sc * X) / np.where(nz, sc, 1.0), 0.0)
    return bf16_round((Db @ X.astype(np.float32)).astype(np.float64))
