"""drgrpo_loss_fwd_bwd_noalloc (the entry point for callers that cannot
allocate: its scratch is a static device array) against the workspace entry
point drgrpo_loss_fwd_bwd, through the C ABI: two calls in a row, the second
with a smaller batch, each bit for bit equal to the workspace call (the same
kernels) and within the oracle's tolerances."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import rl_post_loss_dr_amd as dr
from _cases import compare_dlogits, compare_loss, small_case, to_device_logits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs_small(name):
    cfg, case, x, old, ref, res = small_case(name)
    args = (to_device_logits(x, cfg, DEV), torch.from_numpy(case.tokens).to(DEV), cfg.eos_id,
            torch.from_numpy(case.rewards).to(DEV), torch.from_numpy(old).to(DEV),
            None if ref is None else torch.from_numpy(ref).to(DEV))
    return cfg, args, res


def _inputs_full(name):
    """A benchmark-sized batch generated on the device (no oracle values)."""
    cfg = synth.get_config(name)
    case = synth.make_case(cfg)
    logits = torch.empty((cfg.N, cfg.C, cfg.V), dtype=torch.bfloat16, device=DEV)
    synth.gpu_normal_fill(logits, cfg.seed, synth.S_LOGITS, 0, cfg.logit_std)
    tokens = torch.from_numpy(case.tokens).to(DEV)
    lp = dr.logprobs(logits, tokens).double().cpu().numpy()
    old = torch.from_numpy(synth.perturb(lp, case.old_noise)).to(DEV)
    return cfg, (logits, tokens, cfg.eos_id, torch.from_numpy(case.rewards).to(DEV), old, None)


def _both(cfg, args):
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const)
    loss_w, d_w = dr.loss_fwd_bwd(*args, **kw)
    out_loss = torch.empty((), dtype=torch.float32, device=DEV)
    out_d = torch.empty_like(args[0])
    loss_n, d_n = dr.loss_fwd_bwd_noalloc(*args, out_loss=out_loss, out_dlogits=out_d, **kw)
    torch.cuda.synchronize()
    assert loss_n.data_ptr() == out_loss.data_ptr() and d_n.data_ptr() == out_d.data_ptr()
    return loss_w, d_w, loss_n, d_n


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first call: the benchmark's B=8, G=8, C=256, V=151936 bfloat16 batch
    cfg, args = _inputs_full("qwen_b8g8c256")
    print(f"[noalloc] call 1 {cfg.name} T={cfg.T}", flush=True)
    loss_w, d_w, loss_n, d_n = _both(cfg, args)
    assert np.isfinite(float(loss_w.item()))
    assert float(loss_n.item()) == float(loss_w.item())
    assert torch.equal(d_n.view(torch.int16), d_w.view(torch.int16))
    del args, d_w, d_n
    # second call, smaller: the same static scratch holds the previous call's
    # contents, which must not leak into this one
    for name in ("mini_kl_bf16", "tiny_fp32"):
        cfg, args, res = _inputs_small(name)
        print(f"[noalloc] call {name} T={cfg.T}", flush=True)
        loss_w, d_w, loss_n, d_n = _both(cfg, args)
        assert float(loss_n.item()) == float(loss_w.item())
        view = torch.int16 if d_w.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(d_n.view(view), d_w.view(view))
        compare_loss(cfg, float(loss_n.item()), res)
        compare_dlogits(cfg, d_n.float().cpu().numpy().astype(np.float64).reshape(-1, cfg.V),
                        res.dlogits)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    """A batch whose workspace exceeds the static array returns
    DRGRPO_ERR_SCRATCH_LIMIT before anything is enqueued (the pointers are
    valid device buffers, never touched)."""
    N, C, V = 2048, 1024, 8
    assert dr.workspace_bytes(N, C, V, 8) > dr.NOALLOC_SCRATCH_BYTES
    logits = torch.zeros((N, C, V), dtype=torch.bfloat16, device=DEV)
    dl = torch.zeros_like(logits)
    small = torch.zeros(N * C, dtype=torch.int64, device=DEV)
    p = small.data_ptr()
    rc = dr.lib().drgrpo_loss_fwd_bwd_noalloc(logits.data_ptr(), p, 0, p, p, None, 8, 0.2, 0.0,
                                              1.0, p, dl.data_ptr(), N, C, V, dr.BF16,
                                              ctypes.c_void_p(None))
    assert rc == dr.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert float(dl.float().abs().sum()) == 0.0 and int(small.abs().sum()) == 0
