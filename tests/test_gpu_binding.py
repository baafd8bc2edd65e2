"""The binding refuses caller-supplied outputs and workspaces it cannot hand to
the kernels (a host tensor, a wrong element type or shape, a buffer on the
host or of another type) before anything is launched: the outputs and the
inputs are left untouched.  The Python example of README.md runs as written."""
import pytest
import torch

import rl_post_loss_dr_amd as dr

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _lm_inputs(N=2, C=4, V=64, H=32, G=2):
    hidden = torch.zeros((N * C, H), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=DEV)
    tokens = torch.zeros((N, C), dtype=torch.int64, device=DEV)
    rewards = torch.zeros(N, dtype=torch.float32, device=DEV)
    old = torch.zeros((N, C), dtype=torch.float32, device=DEV)
    return hidden, W, tokens, rewards, old, G


@pytest.mark.parametrize("which,bad,exc", [
    ("out_dhidden", lambda h, W: torch.zeros_like(h, device="cpu"), TypeError),
    ("out_dhidden", lambda h, W: torch.zeros(h.shape, dtype=torch.float32, device=DEV), TypeError),
    ("out_dhidden", lambda h, W: torch.zeros((h.shape[0] - 1, h.shape[1]), dtype=torch.bfloat16,
                                             device=DEV), ValueError),
    ("out_dW", lambda h, W: torch.zeros_like(W, device="cpu"), TypeError),
    ("out_dW", lambda h, W: torch.zeros(W.shape, dtype=torch.float32, device=DEV), TypeError),
    ("out_dW", lambda h, W: torch.zeros((W.shape[0], W.shape[1] + 8), dtype=torch.bfloat16,
                                        device=DEV), ValueError),
    ("workspace", lambda h, W: torch.zeros(1 << 20, dtype=torch.uint8), TypeError),
    ("workspace", lambda h, W: torch.zeros(1 << 18, dtype=torch.float32, device=DEV), TypeError),
])
def test_lmhead_rejects_bad_caller_buffers(which, bad, exc):
    hidden, W, tokens, rewards, old, G = _lm_inputs()
    buf = bad(hidden, W)
    before = buf.clone()
    with pytest.raises(exc):
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, 3, rewards, old, None, G=G, **{which: buf})
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_loss_rejects_bad_workspace_and_devices():
    N, C, V, G = 4, 3, 64, 2
    logits = torch.zeros((N, C, V), dtype=torch.float32, device=DEV)
    tokens = torch.zeros((N, C), dtype=torch.int64, device=DEV)
    rewards = torch.zeros(N, dtype=torch.float32, device=DEV)
    old = torch.zeros((N, C), dtype=torch.float32, device=DEV)
    host_ws = torch.zeros(dr.workspace_bytes(N, C, V, G), dtype=torch.uint8)
    with pytest.raises(TypeError):
        dr.loss_fwd_bwd(logits, tokens, 0, rewards, old, None, G=G, workspace=host_ws)
    with pytest.raises(TypeError):
        dr.loss_fwd_bwd(logits, tokens, 0, rewards, old, None, G=G,
                        workspace=torch.zeros(64, dtype=torch.int32, device=DEV))
    with pytest.raises(TypeError):
        dr.loss_fwd_bwd(logits, tokens, 0, rewards, old.cpu(), None, G=G)
    assert float(host_ws.sum()) == 0


def test_readme_usage_runs():
    """The Python example of README.md, run as written on small inputs: the
    autograd form hands the logits the same dlogits as the direct call, and
    the fused lm_head form returns finite gradients of the right shapes."""
    import os
    import re

    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, flags=re.S).group(1)
    g = torch.Generator(device="cpu").manual_seed(5)
    B, G, C, V, H, eos_id = 2, 8, 8, 4096, 64, 3
    N = B * G
    logits = (torch.randn((N, C, V), generator=g) * 2).to(torch.bfloat16).to(DEV)
    logits.requires_grad_(True)
    tokens = torch.randint(4, V, (N, C), generator=g)
    tokens[0, 2] = eos_id
    tokens = tokens.to(DEV)
    rewards = torch.tensor([1.0, 0.0] * (N // 2), device=DEV)
    hidden = torch.randn((N * C, H), generator=g).to(torch.bfloat16).to(DEV)
    W = (torch.randn((V, H), generator=g) * 0.1).to(torch.bfloat16).to(DEV)
    ns = dict(logits=logits, tokens=tokens, eos_id=eos_id, rewards=rewards, hidden=hidden, W=W)
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    _, dl_direct = dr.loss_fwd_bwd(logits.detach(), tokens, eos_id, rewards,
                                   dr.logprobs(logits.detach(), tokens), G=8)
    assert torch.equal(logits.grad, dl_direct)
    assert torch.isfinite(ns["loss"]).item()
    assert ns["dhidden"].shape == hidden.shape and ns["dW"].shape == W.shape
    assert torch.isfinite(ns["dhidden"].float()).all() and torch.isfinite(ns["dW"].float()).all()
