"""GPU parity of the normalisation variants ("Making Dr GRPO go brrr",
sections "GRPO" and "Dr. GRPO": GRPO's group-standardised advantage and
per-response mean, and the token mean) against the oracle, element by
element, plus the extra rollout counters."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rl_post_loss_dr_amd as dr
from _cases import compare_dlogits, dlogits_to_f64, exempt_rows, f32, lm_case, to_device_logits, tol
from _lmcheck import check_dW, check_dhidden

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

VARIANTS = [(dr.ADV_ZSCORE, dr.AGG_SEQ_MEAN), (dr.ADV_CENTER, dr.AGG_TOKEN_MEAN),
            (dr.ADV_ZSCORE, dr.AGG_TOKEN_SUM), (dr.ADV_CENTER, dr.AGG_SEQ_MEAN)]


def _case(name, adv_mode, agg, kappa=None):
    cfg = synth.get_config(name)
    case = synth.make_case(cfg)
    x = case.logits_rows(np.arange(cfg.T))
    _, logp, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    logp = logp.reshape(cfg.N, cfg.C)
    old = synth.perturb(logp, case.old_noise)
    ref = None if case.ref_noise is None else synth.perturb(logp, case.ref_noise)
    k = f32(kappa or cfg.norm_const)
    res = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                              f32(cfg.eps), f32(cfg.beta), k, adv_mode=adv_mode, agg=agg)
    return cfg, case, x, old, ref, res, k


@pytest.mark.parametrize("name", ["tiny_fp32", "mini_kl_bf16", "clip_heavy_bf16", "odd_v_f32",
                                  "ragged_bf16"])
@pytest.mark.parametrize("adv_mode,agg", VARIANTS)
@pytest.mark.parametrize("kappa_one", [False, True])
def test_variant_parity_small(name, adv_mode, agg, kappa_one):
    print(f"case {name} adv_mode={adv_mode} agg={agg} kappa_one={kappa_one}", flush=True)
    cfg, case, x, old, ref, res, k = _case(name, adv_mode, agg, 1.0 if kappa_one else None)
    aux = {}
    counts = torch.empty(2, dtype=torch.int64, device=DEV)
    loss, d = dr.loss_fwd_bwd(
        to_device_logits(x, cfg, DEV), torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
        torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV),
        None if ref is None else torch.from_numpy(ref).to(DEV), G=cfg.G, eps=cfg.eps,
        beta=cfg.beta, norm_const=k, aux=aux, adv_mode=adv_mode, agg=agg, out_counts=counts)
    torch.cuda.synchronize()
    # advantages: bit-exact binary32 (sample std, correctly rounded sqrt and division)
    assert np.array_equal(aux["adv"].cpu().numpy().view(np.uint32), res.adv.view(np.uint32))
    assert len(exempt_rows(cfg, res, old)) == 0
    st = aux["stats"].cpu().numpy()
    mask = np.arange(cfg.C)[None, :] < res.len[:, None]
    act = mask & ((res.adv[:, None] != 0) | (cfg.beta != 0))
    ct = counts.cpu().numpy()
    assert ct[0] == res.len.sum() and ct[1] == act.sum()
    assert st[2] == res.stats[0] and st[3] == res.stats[1]
    # loss: relative to the same aggregation of |lambda| when it cancels
    div = oracle.row_divisor(res.len, k, agg)
    scale = float((np.abs(res.lam).sum(axis=1) / div).sum())
    L = float(loss.item())
    t = tol(cfg)
    ref_scale = abs(res.loss) if scale / max(abs(res.loss), 1e-300) <= 1e4 else scale
    assert abs(L - res.loss) <= t["loss_rel"] * ref_scale, (L, res.loss, scale)
    got = dlogits_to_f64(d)
    compare_dlogits(cfg, got, res.dlogits)
    assert (got[res.coef.reshape(-1) == 0] == 0).all()


def test_zscore_advantage_entry_point_bit_exact():
    rng = np.random.default_rng(11)
    for G in (1, 2, 3, 5, 8, 16):
        r = rng.choice(np.array([0, 0.25, 0.5, 0.75, 1, 0.1, 0.3], np.float32), size=64 * G)
        r[:G] = 0.5  # a uniform group
        if G > 1:
            r[G:2 * G] = np.float32(0.1)
            r[2 * G] = np.float32(0.1) + np.float32(1e-7)  # nearly uniform: huge advantages
        adv, cnt = dr.group_advantage(torch.from_numpy(r).to(DEV), G, dr.ADV_ZSCORE)
        want = oracle.group_advantage(r, G, oracle.ADV_ZSCORE)
        assert np.array_equal(adv.cpu().numpy().view(np.uint32), want.view(np.uint32)), G
        assert int(cnt.item()) == oracle.nocontrast_groups(r, G)


@pytest.mark.parametrize("adv_mode,agg", [(dr.ADV_ZSCORE, dr.AGG_SEQ_MEAN),
                                          (dr.ADV_CENTER, dr.AGG_TOKEN_MEAN)])
def test_lmhead_variant_parity(adv_mode, agg):
    """The fused lm_head path with the GRPO normalisations / token mean."""
    from oracle import lmhead

    cfg, case, hb, Wb, old, ref, _ = lm_case("lmhead_multi")
    t = lmhead.full(hb, Wb, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                    f32(cfg.eps), f32(cfg.beta), f32(cfg.norm_const), adv_mode, agg)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(DEV)

    loss, dh, dW = dr.lmhead_loss_fwd_bwd(
        dev_bf16(hb), dev_bf16(Wb), torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
        torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV),
        None if ref is None else torch.from_numpy(ref).to(DEV), G=cfg.G, eps=cfg.eps,
        beta=cfg.beta, norm_const=cfg.norm_const, adv_mode=adv_mode, agg=agg)
    torch.cuda.synchronize()
    assert abs(float(loss.item()) - t["loss"]) <= 2e-3 * abs(t["loss"])
    h64 = lmhead.bf16_to_f64(hb)
    W64 = lmhead.bf16_to_f64(Wb)
    tok = case.tokens.reshape(-1)
    act = t["active_rows"]
    f64 = lambda g: g.float().cpu().numpy().astype(np.float64)  # noqa: E731
    check_dhidden(f64(dh), t["dlogits"], W64, t["coef"], tok)
    check_dW(f64(dW), t["dlogits"][act], h64[act], np.isin(np.arange(cfg.V), tok[act]))
