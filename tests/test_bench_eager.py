"""The plain eager-PyTorch formulation that bench.py times beside the fused
call (context only) computes the method: in binary64 on the CPU its loss and
its autograd dlogits equal the oracle's on small cases, with and without the
KL term, with clipped tokens, EOS at the first position and rows without EOS.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth


@pytest.mark.parametrize("name", ["tiny_fp32", "clip_heavy_f32", "mini_kl_bf16"])
def test_eager_formulation_matches_oracle(name):
    cfg = synth.get_config(name)
    case = synth.make_case(cfg)
    x = case.logits_rows_f32(np.arange(cfg.T)).astype(np.float64).reshape(cfg.N, cfg.C, cfg.V)
    ref_res = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards,
                                  np.zeros((cfg.N, cfg.C), np.float32), None, cfg.G, cfg.eps,
                                  0.0, cfg.norm_const, want_dlogits=False)
    old = synth.perturb(ref_res.logp, case.old_noise)
    ref = None if case.ref_noise is None else synth.perturb(ref_res.logp, case.ref_noise)
    want = oracle.loss_fwd_bwd(x, case.tokens, cfg.eos_id, case.rewards, old, ref, cfg.G,
                               cfg.eps, cfg.beta, cfg.norm_const)

    xt = torch.from_numpy(x).requires_grad_(True)
    tok = torch.from_numpy(case.tokens)
    lp = torch.log_softmax(xt, dim=-1).gather(-1, tok.unsqueeze(-1)).squeeze(-1)
    loss = bench._eager_terms(lp, tok, cfg.eos_id, torch.from_numpy(case.rewards).double(),
                              torch.from_numpy(old).double(),
                              None if ref is None else torch.from_numpy(ref).double(),
                              cfg.G, cfg.eps, cfg.beta, cfg.norm_const)
    loss.backward()
    assert loss.item() == pytest.approx(want.loss, rel=1e-9, abs=1e-12)
    got = xt.grad.numpy().reshape(cfg.T, cfg.V)
    scale = np.abs(want.dlogits).max()
    assert scale > 0
    np.testing.assert_allclose(got, want.dlogits, rtol=0, atol=1e-9 * scale)
