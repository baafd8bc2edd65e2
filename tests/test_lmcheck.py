"""The fused lm_head gradient checker can fail: it accepts the oracle's
gradients carried through the GPU's precision path (dlogits as bfloat16
exponentials times a per-token factor, for dW the hidden rows scaled and
rounded to bfloat16, binary32 products, bfloat16 results, emulated on the
CPU) and rejects the
same arrays with one part of the gradient wrong - the vocabulary rows of dW
that no active token sampled zeroed or scaled by 1.01, one such row zeroed,
dhidden's softmax part dropped or scaled, the sampled dW rows or dhidden
scaled by 1.01.  CPU only."""
import numpy as np
import pytest

from oracle import lmhead
from _cases import lm_case
from _lmcheck import bf16_round, check_dhidden, check_dW, emulate

CASES = ["lmhead_mini", "lmhead_multi", "lmhead_chunks3"]


def _pieces(name):
    cfg, case, hb, Wb, old, ref, t = lm_case(name)
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    D = t["dlogits"]
    act = t["active_rows"]
    Ha = h64[act]
    Dc = D[act]
    sampled = np.isin(np.arange(cfg.V), tok[act])
    return cfg, h64, W64, tok, D, Dc, Ha, sampled, t


@pytest.mark.parametrize("name", CASES)
def test_checker_accepts_gpu_precision(name):
    cfg, h64, W64, tok, D, Dc, Ha, sampled, t = _pieces(name)
    dh = emulate(D, W64)
    dW = emulate(Dc.T, Ha, t["coef"][t["active_rows"]])
    r1 = check_dhidden(dh, D, W64, t["coef"], tok)
    r2 = check_dW(dW, Dc, Ha, sampled)
    print(name, r1, r2)
    # the parts the checker must see exist in every case
    assert "softmax" in r1 and "dW unsampled rows" in r2 and "dW sampled rows" in r2


@pytest.mark.parametrize("name", CASES)
def test_checker_rejects_wrong_dW_parts(name):
    cfg, h64, W64, tok, D, Dc, Ha, sampled, t = _pieces(name)
    dW = emulate(Dc.T, Ha, t["coef"][t["active_rows"]])
    uns = np.flatnonzero(~sampled)
    samp = np.flatnonzero(sampled)
    # nonzero unsampled rows: the ones a wrong kernel could silently zero
    live = uns[np.abs(dW[uns]).max(axis=1) > 0]
    assert live.size > 0
    variants = {}
    z = dW.copy(); z[uns] = 0.0; variants["unsampled rows zeroed"] = z
    s = dW.copy(); s[uns] = bf16_round(dW[uns] * 1.01); variants["unsampled rows x1.01"] = s
    one = dW.copy(); one[live[len(live) // 2]] = 0.0; variants["one unsampled row zeroed"] = one
    ss = dW.copy(); ss[samp] = bf16_round(dW[samp] * 1.01); variants["sampled rows x1.01"] = ss
    for label, bad in variants.items():
        with pytest.raises(AssertionError):
            check_dW(bad, Dc, Ha, sampled)
        print(name, label, "rejected")


@pytest.mark.parametrize("name", CASES)
def test_checker_rejects_wrong_dhidden_parts(name):
    cfg, h64, W64, tok, D, Dc, Ha, sampled, t = _pieces(name)
    coef = t["coef"]
    live = coef != 0
    dh = emulate(D, W64)
    # the softmax part dropped: only the sampled token's -coef entry reaches W
    Dh = np.zeros_like(D)
    Dh[np.flatnonzero(live), tok[live]] = -coef[live]
    variants = {"softmax part dropped": emulate(Dh, W64)}
    # the softmax part scaled by 0.9 (the sampled token's term kept)
    D9 = 0.9 * D
    D9[np.flatnonzero(live), tok[live]] = D[np.flatnonzero(live), tok[live]] - 0.1 * coef[live]
    variants["softmax part x0.9"] = emulate(D9, W64)
    variants["dhidden x1.01"] = bf16_round(dh * 1.01)
    # one active row zeroed
    z = dh.copy(); z[np.flatnonzero(live)[0]] = 0.0; variants["one row zeroed"] = z
    for label, bad in variants.items():
        with pytest.raises(AssertionError):
            check_dhidden(bad, D, W64, coef, tok)
        print(name, label, "rejected")
