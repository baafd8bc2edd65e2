"""GPU parity of the fused Dr. GRPO loss against the CPU oracle, element by
element, on seeded inputs small enough for the oracle to finish in seconds
(several vocabulary tiles, ragged tails, every edge case the method has)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rl_post_loss_dr_amd as dr
from _cases import (compare_dlogits, compare_loss, dlogits_to_f64, exempt_rows, f32, small_case,
                    to_device_logits)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")

SMALL = ["tiny_fp32", "mini_bf16", "mini_kl_bf16", "ragged_bf16", "odd_v_f32", "odd_v_bf16",
         "clip_heavy_f32", "clip_heavy_bf16", "big_v_f32", "big_v_bf16", "no_eos_id",
         "many_seq_bf16", "many_seq_c1_bf16", "ticket_v4_f32", "ticket_odd_bf16"]


def _run(cfg, case, x, old, ref, kappa=None, out=None, aux=None, logits=None):
    if logits is None:
        logits = to_device_logits(x, cfg, DEV)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    rewards = torch.from_numpy(case.rewards).to(DEV)
    lo = torch.from_numpy(old).to(DEV)
    lr = None if ref is None else torch.from_numpy(ref).to(DEV)
    loss, d = dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, lo, lr, G=cfg.G, eps=cfg.eps,
                              beta=cfg.beta, norm_const=kappa or cfg.norm_const, out_dlogits=out,
                              aux=aux)
    torch.cuda.synchronize()
    return float(loss.item()), d


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("kappa_one", [False, True])
def test_parity_small(name, kappa_one):
    print(f"case {name} kappa_one={kappa_one}", flush=True)
    cfg0 = synth.get_config(name)
    kappa = 1.0 if kappa_one else None
    cfg, case, x, old, ref, res = small_case(name, kappa)
    aux = {}
    loss, d = _run(cfg, case, x, old, ref, kappa=kappa, aux=aux)
    # integer and index work: bit-exact
    assert np.array_equal(aux["len"].cpu().numpy(), res.len)
    assert np.array_equal(aux["mask"].cpu().numpy(),
                          (np.arange(cfg.C)[None, :] < res.len[:, None]).astype(np.uint8))
    assert np.array_equal(aux["adv"].cpu().numpy().view(np.uint32), res.adv.view(np.uint32))
    st = aux["stats"].cpu().numpy()
    assert st[0] == res.nocontrast and st[1] == res.truncated
    ex = exempt_rows(cfg, res, old)
    assert len(ex) == 0, f"{len(ex)} tokens on a clip boundary"
    assert st[2] == res.stats[0] and st[3] == res.stats[1]
    # floats
    compare_loss(cfg, loss, res)
    got = dlogits_to_f64(d)
    compare_dlogits(cfg, got, res.dlogits)
    inactive = (res.coef.reshape(-1) == 0)
    assert (got[inactive] == 0).all()
    lp = aux["logp"].cpu().numpy().astype(np.float64)
    mask = np.arange(cfg.C)[None, :] < res.len[:, None]
    act = mask & ((res.adv[:, None] != 0) | (cfg.beta != 0))
    assert act.any()
    assert np.abs(lp[act] - res.logp[act]).max() <= (2e-6 if cfg.dtype == "f32" else 2e-5) * \
        max(1.0, np.abs(res.logp[act]).max())
    assert (lp[~act] == 0).all()
    tl = aux["tok_loss"].cpu().numpy().astype(np.float64)
    assert np.allclose(tl, res.lam, rtol=1e-5, atol=1e-7)
    assert cfg0 is not None


def test_determinism_and_inplace():
    cfg, case, x, old, ref, res = small_case("mini_kl_bf16")
    l1, d1 = _run(cfg, case, x, old, ref)
    l2, d2 = _run(cfg, case, x, old, ref)
    assert l1 == l2 and torch.equal(d1, d2)
    logits = to_device_logits(x, cfg, DEV)
    l3, d3 = _run(cfg, case, x, old, ref, out=logits, logits=logits)
    assert d3.data_ptr() == logits.data_ptr()
    assert l3 == l1 and torch.equal(d3, d1)


def test_inplace_streaming_rows():
    """In place on rows longer than one register tile (re-read pass)."""
    cfg, case, x, old, ref, res = small_case("big_v_f32")
    l1, d1 = _run(cfg, case, x, old, ref)
    logits = to_device_logits(x, cfg, DEV)
    l2, d2 = _run(cfg, case, x, old, ref, out=logits, logits=logits)
    assert l1 == l2 and torch.equal(d1, d2)


def test_step0_identity_on_gpu():
    """logp_old from the library's own forward pass: the ratio is exactly 1
    and the loss is -sum_i A_i |o_i| / kappa ("The loss": inner step 0)."""
    cfg, case, x, old, ref, res = small_case("mini_bf16")
    logits = to_device_logits(x, cfg, DEV)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    lp = dr.logprobs(logits, tokens)
    loss, d = dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, torch.from_numpy(case.rewards).to(DEV),
                              lp, None, G=cfg.G, eps=cfg.eps, beta=0.0,
                              norm_const=cfg.norm_const, aux=(aux := {}))
    want = -float((res.adv.astype(np.float64) * res.len).sum()) / f32(cfg.norm_const)
    scale = float((np.abs(res.adv.astype(np.float64)) * res.len).sum()) / f32(cfg.norm_const)
    # logp_old is binary32: the ratio is 1 to within its rounding (~5e-7)
    assert abs(float(loss.item()) - want) <= 1e-6 * scale
    st = aux["stats"].cpu().numpy()
    assert st[2] == 0 and st[3] == 0


@pytest.mark.parametrize("name", ["tiny_fp32", "mini_bf16", "odd_v_f32", "odd_v_bf16",
                                  "big_v_bf16"])
def test_logprobs_forward_only(name):
    cfg, case, x, old, ref, res = small_case(name)
    logits = to_device_logits(x, cfg, DEV)
    lp = dr.logprobs(logits, torch.from_numpy(case.tokens).to(DEV)).cpu().numpy()
    _, want, _ = oracle.row_logprob(x, case.tokens.reshape(-1))
    err = np.abs(lp.astype(np.float64).reshape(-1) - want).max()
    assert err <= (2e-6 if cfg.dtype == "f32" else 2e-5) * max(1.0, np.abs(want).max()), err


def test_mask_and_advantage_entry_points():
    rng = np.random.default_rng(5)
    for C in (1, 5, 63, 64, 65, 200, 1024):
        tok = rng.integers(0, 4, size=(37, C)).astype(np.int64)
        ln, mk = dr.completion_mask(torch.from_numpy(tok).to(DEV), 0)
        assert np.array_equal(ln.cpu().numpy(), oracle.completion_len(tok, 0))
        assert np.array_equal(mk.cpu().numpy(), oracle.completion_mask(tok, 0))
    for G in (1, 2, 8, 16):
        r = (rng.integers(0, 5, size=16 * G) / 4).astype(np.float32)
        r[:G] = 0.5
        adv, cnt = dr.group_advantage(torch.from_numpy(r).to(DEV), G)
        assert np.array_equal(adv.cpu().numpy().view(np.uint32),
                              oracle.group_advantage(r, G).view(np.uint32))
        assert int(cnt.item()) == oracle.nocontrast_groups(r, G)


def test_bernoulli_nocontrast_count_matches_cpu():
    """Check (d) on the device: the GPU's no-contrast count of 10^6 generated
    Bernoulli(0.05) groups of 8 equals the oracle's count exactly."""
    M, G = 1_000_000, 8
    r = (synth.uniform01(99, synth.S_REWARDS, np.arange(M * G)) < 0.05).astype(np.float32)
    _, cnt = dr.group_advantage(torch.from_numpy(r).to(DEV), G)
    assert int(cnt.item()) == oracle.nocontrast_groups(r, G)


def test_token_out_of_range_sets_status():
    cfg, case, x, old, ref, res = small_case("tiny_fp32")
    logits = to_device_logits(x, cfg, DEV)
    tok = case.tokens.copy()
    # a bad id at a masked position is ignored
    masked = np.argwhere(np.arange(cfg.C)[None, :] >= res.len[:, None])
    i, t = masked[0]
    tok[i, t] = cfg.V + 5
    ws = dr.make_workspace(cfg.N, cfg.C, cfg.V, cfg.G, DEV)
    args = (torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV), None)
    loss, d = dr.loss_fwd_bwd(logits, torch.from_numpy(tok).to(DEV), cfg.eos_id, *args, G=cfg.G,
                              workspace=ws)
    assert dr.device_status(ws) == dr.OK
    assert float(loss.item()) == pytest.approx(res.loss, rel=1e-5)
    # a bad id at a counted position poisons the loss and that row
    i5 = int(np.flatnonzero(res.len > 1)[0])
    row = i5 * cfg.C + 1
    tok2 = case.tokens.copy().reshape(-1)
    tok2[row] = -3
    loss, d = dr.loss_fwd_bwd(logits, torch.from_numpy(tok2.reshape(cfg.N, cfg.C)).to(DEV),
                              cfg.eos_id, *args, G=cfg.G, workspace=ws)
    assert dr.device_status(ws) == dr.ERR_TOKEN_RANGE
    assert np.isnan(float(loss.item()))
    dd = d.reshape(-1, cfg.V)
    assert torch.isnan(dd[row]).all()
    # the next good call clears the status word
    dr.loss_fwd_bwd(logits, torch.from_numpy(case.tokens).to(DEV), cfg.eos_id, *args, G=cfg.G,
                    workspace=ws)
    assert dr.device_status(ws) == dr.OK


def test_token_out_of_range_full_size_rows():
    """The same rule on full-size rows (V = 151,936, the 1024-thread kernel and
    its ticket order): an id outside [0, V) is ignored at a masked position,
    and at a counted position, of a completion with or without reward
    contrast, makes the loss NaN, that row NaN and the status word report it;
    every other dlogits row is bit for bit the good call's."""
    cfg, case, x, old, ref, res = small_case("mini_bf16")
    logits = to_device_logits(x, cfg, DEV)
    args = (torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV), None)
    ws = dr.make_workspace(cfg.N, cfg.C, cfg.V, cfg.G, DEV)

    def run(tok):
        loss, d = dr.loss_fwd_bwd(logits, torch.from_numpy(tok).to(DEV), cfg.eos_id, *args,
                                  G=cfg.G, workspace=ws)
        torch.cuda.synchronize()
        return float(loss.item()), d.reshape(-1, cfg.V).view(torch.int16).cpu().numpy(), \
            dr.device_status(ws)

    loss0, d0, st0 = run(case.tokens)
    assert st0 == dr.OK
    lens, adv = res.len, res.adv
    # completions that end in an EOS with room before it: positions before the
    # EOS are counted and replacing their id leaves every length unchanged
    act_seq = [i for i in range(cfg.N) if adv[i] != 0 and 3 <= lens[i] < cfg.C]
    zero_seq = [i for i in range(cfg.N) if adv[i] == 0 and 3 <= lens[i] < cfg.C]
    assert act_seq and zero_seq
    # masked position (past the EOS): ignored
    i = act_seq[0]
    tok = case.tokens.copy()
    tok[i, lens[i]] = cfg.V + 5
    loss, d, st = run(tok)
    assert st == dr.OK and loss == loss0 and np.array_equal(d, d0)
    # counted positions, with and without reward contrast, several bad ids
    for i, tt, bad in ((act_seq[0], lens[act_seq[0]] - 2, -3), (act_seq[-1], 0, cfg.V),
                       (zero_seq[0], 1, 1 << 40)):
        tok = case.tokens.copy()
        tok[i, tt] = bad
        loss, d, st = run(tok)
        row = i * cfg.C + tt
        print(f"completion {i} position {tt} id {bad}", flush=True)
        assert st == dr.ERR_TOKEN_RANGE
        assert np.isnan(loss)
        got_row = d[row].view(np.uint16)
        assert ((got_row & 0x7F80) == 0x7F80).all() and ((got_row & 0x007F) != 0).all()
        others = np.ones(d.shape[0], bool)
        others[row] = False
        assert np.array_equal(d[others], d0[others])
    loss, d, st = run(case.tokens)
    assert st == dr.OK and loss == loss0 and np.array_equal(d, d0)


def test_nan_logits_propagate_only_from_counted_rows():
    cfg, case, x, old, ref, res = small_case("tiny_fp32")
    x2 = x.copy()
    act = np.flatnonzero(res.coef.reshape(-1) != 0)
    masked = np.flatnonzero((np.arange(cfg.C)[None, :] >= res.len[:, None]).reshape(-1))
    x2[masked] = np.nan
    l_ok, _ = _run(cfg, case, x2, old, ref)
    assert l_ok == pytest.approx(res.loss, rel=1e-5)
    x2[act[3], 7] = np.nan
    l_bad, _ = _run(cfg, case, x2, old, ref)
    assert np.isnan(l_bad)


def test_autograd_wrapper():
    cfg, case, x, old, ref, res = small_case("tiny_fp32")
    logits = to_device_logits(x, cfg, DEV).requires_grad_(True)
    loss = dr.DrGRPOLoss.apply(logits, torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
                               torch.from_numpy(case.rewards).to(DEV),
                               torch.from_numpy(old).to(DEV), None, cfg.G, cfg.eps, 0.0,
                               cfg.norm_const)
    (3.0 * loss).backward()
    g = logits.grad.detach().cpu().numpy().astype(np.float64).reshape(cfg.T, cfg.V)
    assert np.abs(g - 3.0 * res.dlogits).max() <= 3e-5
    # seed 1 (loss.backward()): the gradient is dlogits itself, bit for bit
    logits.grad = None
    args = (torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
            torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV), None, cfg.G,
            cfg.eps, 0.0, cfg.norm_const)
    dr.DrGRPOLoss.apply(logits, *args).backward()
    _, d = dr.loss_fwd_bwd(logits.detach(), *args[:4], G=cfg.G, eps=cfg.eps, beta=0.0,
                           norm_const=cfg.norm_const)
    assert torch.equal(logits.grad, d)


def test_generator_bits_match_cpu():
    """The device generator writes exactly the host generator's values."""
    for dtype, torch_dt in ((synth.F32, torch.float32), (synth.BF16, torch.bfloat16)):
        n = 1_000_003
        t = torch.empty(n, dtype=torch_dt, device=DEV)
        synth.gpu_normal_fill(t, 1234, synth.S_LOGITS, 77, 2.0)
        torch.cuda.synchronize()
        host = synth.cpu_normal(1234, synth.S_LOGITS, 77, n, 2.0, dtype)
        got = t.cpu()
        got = got.numpy() if dtype == synth.F32 else got.view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got.view(np.uint8), host.view(np.uint8))
