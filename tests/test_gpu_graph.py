"""The loss entry points captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed, as a training or rollout loop would issue them: every replay equals
the eager call bit for bit, with eager work and synchronisations between
replays and the outputs overwritten before each replay.  The library only
launches kernels (no memset, no host synchronisation; the workspace state is
cleared by its own kernels: the row kernel's ticket counters by k_prep, at
320 completions also by k_plan), which is what makes the capture valid."""
import numpy as np
import pytest
import torch

import rl_post_loss_dr_amd as dr
from _cases import lm_case, scaled_bf16_rows, small_case, to_device_logits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns the
    graph and what the captured call returned."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = fn()
    return graph, res


def _bits_to_dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("name", ["tiny_fp32", "mini_kl_bf16", "ragged_bf16", "many_seq_bf16"])
def test_loss_graph_replay(name):
    print(f"case {name}", flush=True)
    cfg, case, x, old, ref, _ = small_case(name)
    logits = to_device_logits(x, cfg, DEV)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    rewards = torch.from_numpy(case.rewards).to(DEV)
    lo = torch.from_numpy(old).to(DEV)
    lr = None if ref is None else torch.from_numpy(ref).to(DEV)
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const)
    ws = dr.make_workspace(cfg.N, cfg.C, cfg.V, cfg.G, DEV)
    loss_e, d_e = dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, lo, lr, workspace=ws, **kw)
    loss_e, d_e = loss_e.clone(), d_e.clone()
    d_g = torch.empty_like(d_e)
    ws_g = dr.make_workspace(cfg.N, cfg.C, cfg.V, cfg.G, DEV)
    graph, (loss_g, _) = _capture(lambda: dr.loss_fwd_bwd(
        logits, tokens, cfg.eos_id, rewards, lo, lr, out_dlogits=d_g, workspace=ws_g, **kw))
    flipped = rewards.flip(0).contiguous()
    for _ in range(4):
        d_g.fill_(1.0)
        loss_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss_e)
        assert torch.equal(d_g, d_e)
        # eager work between replays, on the other workspace
        dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, flipped, lo, lr, workspace=ws, **kw)
        torch.cuda.synchronize()
    assert dr.device_status(ws_g) == dr.OK


def test_lmhead_graph_replay():
    """Fused lm_head loss (compaction, chunked products, device-side active
    count) and its forward-only log-probs, each replayed from a graph."""
    cfg, case, hb, Wb, old, ref, _ = lm_case("lmhead_multi")
    hidden, W = _bits_to_dev(hb), _bits_to_dev(Wb)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    rewards = torch.from_numpy(case.rewards).to(DEV)
    lo = torch.from_numpy(old).to(DEV)
    lr = None if ref is None else torch.from_numpy(ref).to(DEV)
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const)
    ws_bytes = dr.lmhead_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H, cfg.G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    loss_e, dh_e, dW_e = dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, lo, lr,
                                                 workspace=ws, **kw)
    loss_e, dh_e, dW_e = loss_e.clone(), dh_e.clone(), dW_e.clone()
    lp_e = dr.lmhead_logprobs(hidden, W, tokens, cfg.eos_id).clone()

    dh_g, dW_g = torch.empty_like(dh_e), torch.empty_like(dW_e)
    ws_g = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    graph, (loss_g, _, _) = _capture(lambda: dr.lmhead_loss_fwd_bwd(
        hidden, W, tokens, cfg.eos_id, rewards, lo, lr, out_dhidden=dh_g, out_dW=dW_g,
        workspace=ws_g, **kw))
    ws_lp = torch.empty(dr.lmhead_logprobs_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H),
                        dtype=torch.uint8, device=DEV)
    graph_lp, lp_g = _capture(lambda: dr.lmhead_logprobs(hidden, W, tokens, cfg.eos_id,
                                                         workspace=ws_lp))
    for _ in range(3):
        dh_g.fill_(1.0)
        dW_g.fill_(1.0)
        loss_g.fill_(float("nan"))
        lp_g.fill_(1.0)
        graph.replay()
        graph_lp.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss_e)
        assert torch.equal(dh_g, dh_e) and torch.equal(dW_g, dW_e)
        assert torch.equal(lp_g, lp_e)
        # eager work between replays, on the other workspace
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards.flip(0).contiguous(), lo,
                               lr, workspace=ws, **kw)
        torch.cuda.synchronize()


def test_lmhead_graph_replay_rows_beyond_reference():
    """The fused lm_head's flagged-row pass inside captured graphs (the loss
    and the forward-only log-probs): each graph replayed while its hidden
    states alternate, in place, between inputs that put 9 of 20 active rows
    beyond their reference (every other token's row scaled by 32) and inputs
    that put none there; every replay equals the eager call on the same
    inputs bit for bit, so the flag and the row marks are cleared by the
    library's own kernels on every call."""
    import synth
    from oracle import lmhead

    cfg, case, hb, Wb, _, _, _ = lm_case("lmhead_multi")
    hb_far = scaled_bf16_rows(hb, np.arange(0, cfg.T, 2), 32.0)
    W = _bits_to_dev(Wb)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    rewards = torch.from_numpy(case.rewards).to(DEV)
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const)
    ws_bytes = dr.lmhead_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H, cfg.G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    inputs = {}
    for k, bits in (("near", hb), ("far", hb_far)):
        # old / reference log-probs near each input's own (the policy's)
        _, lp = lmhead.token_rows(lmhead.bf16_to_f64(bits), lmhead.bf16_to_f64(Wb),
                                  case.tokens.reshape(-1), np.arange(cfg.T))
        lp = lp.reshape(cfg.N, cfg.C)
        inputs[k] = (_bits_to_dev(bits), torch.from_numpy(synth.perturb(lp, case.old_noise)).to(DEV),
                     torch.from_numpy(synth.perturb(lp, case.ref_noise)).to(DEV))
    want = {}
    for k, (h, lo, lr) in inputs.items():
        l, dh, dW = dr.lmhead_loss_fwd_bwd(h, W, tokens, cfg.eos_id, rewards, lo, lr, workspace=ws,
                                           **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(l) and bool(torch.isfinite(dh.float()).all()), k
        want[k] = (l.clone(), dh.clone(), dW.clone())
    assert not torch.equal(want["near"][2], want["far"][2])
    hidden, lo, lr = (x.clone() for x in inputs["near"])
    dh_g, dW_g = torch.empty_like(hidden), torch.empty_like(W)
    ws_g = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    graph, (loss_g, _, _) = _capture(lambda: dr.lmhead_loss_fwd_bwd(
        hidden, W, tokens, cfg.eos_id, rewards, lo, lr, out_dhidden=dh_g, out_dW=dW_g,
        workspace=ws_g, **kw))
    # the forward-only log-probs of the same inputs, also from a graph
    lp_want = {k: dr.lmhead_logprobs(h, W, tokens, cfg.eos_id).clone() for k, (h, _, _) in
               inputs.items()}
    torch.cuda.synchronize()
    ws_lp = torch.empty(dr.lmhead_logprobs_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H),
                        dtype=torch.uint8, device=DEV)
    graph_lp, lp_g = _capture(lambda: dr.lmhead_logprobs(hidden, W, tokens, cfg.eos_id,
                                                         workspace=ws_lp))
    for k in ["far", "near", "far", "near", "far"]:
        for dst, src in zip((hidden, lo, lr), inputs[k]):
            dst.copy_(src)
        lp_g.fill_(1.0)
        torch.cuda.synchronize()
        graph_lp.replay()
        torch.cuda.synchronize()
        assert torch.equal(lp_g, lp_want[k]), k
        dh_g.fill_(1.0)
        dW_g.fill_(1.0)
        loss_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        l, dh, dW = want[k]
        assert torch.equal(loss_g, l), k
        assert torch.equal(dh_g, dh) and torch.equal(dW_g, dW), k
