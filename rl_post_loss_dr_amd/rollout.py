"""The rollout step the decode attention serves, integrated: one decode step of
a Qwen2.5-0.5B-shaped policy on a (B*G, 1, hidden) input with a growing KV
cache ("Making Dr GRPO go brrr", section "What is RL post-training, and why is
it slow": rollout is one forward pass per generated token, and a decode
kernel's standalone win has to survive integration into that loop).

The weights are random (no checkpoint is used or needed: the step's cost does
not depend on their values).  Every op but the attention block is plain PyTorch
(the projections are hipBLASLt GEMMs); the attention block (rotary
embedding of the new query and key, their append to the layer's cache, and
attention over it) is one library call.  The whole step reads the
positions from the device and writes the new keys and values with indexed
stores, so it can be captured once into a HIP graph and replayed per token, as
a rollout loop would run it.

Architecture (the published Qwen2.5-0.5B shape): 24 layers, hidden 896,
14 query heads and 2 key/value heads of size 64, biases on the q/k/v
projections, rotary position embedding (rotate-half form, base 1e6), RMSNorm
(eps 1e-6), SiLU-gated MLP of width 4864, vocabulary 151936 with the output
projection tied to the embedding; greedy next token.
"""
from __future__ import annotations

import dataclasses
import math

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class PolicyShape:
    layers: int = 24
    hidden: int = 896
    heads: int = 14
    kv_heads: int = 2
    head_dim: int = 64
    inter: int = 4864
    vocab: int = 151936
    rope_base: float = 1.0e6
    eps: float = 1.0e-6


QWEN25_05B = PolicyShape()


class DecodePolicy:
    """Random-init policy with a [S, Hkv, Lmax, D] bfloat16 KV cache per layer.

    step(tok, pos) runs one decode step for all S sequences: tok [S] int64 is
    each sequence's newest token, pos [S] int32 its position (the number of
    positions already cached); the step writes that token's keys and values
    at pos, attends over pos + 1 positions, and returns the logits [S, V]
    (bfloat16) and the greedy next tokens [S] int64.  attention="library" runs
    the rotary embedding, cache append and attention as one library call
    (drgrpo_decode_attention_rope); "library_unfused" the rotary embedding and
    append in PyTorch around drgrpo_decode_attention; "reference" those
    PyTorch steps around a binary32 softmax attention written out in PyTorch
    (for checks, not for timing)."""

    def __init__(self, shape: PolicyShape, S: int, Lmax: int, seed: int, device,
                 std: float = 0.02):
        self.shape, self.S, self.Lmax, self.device = shape, S, Lmax, device
        sh = shape
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def rnd(*size, scale=std):
            return (torch.randn(*size, generator=g, device=device, dtype=torch.float32)
                    * scale).to(torch.bfloat16)

        nq, nkv = sh.heads * sh.head_dim, sh.kv_heads * sh.head_dim
        self.embed = rnd(sh.vocab, sh.hidden)
        self.layers = []
        for _ in range(sh.layers):
            self.layers.append(dict(
                ln1=torch.ones(sh.hidden, dtype=torch.bfloat16, device=device),
                wqkv=rnd(nq + 2 * nkv, sh.hidden), bqkv=rnd(nq + 2 * nkv),
                wo=rnd(sh.hidden, nq),
                ln2=torch.ones(sh.hidden, dtype=torch.bfloat16, device=device),
                wgu=rnd(2 * sh.inter, sh.hidden), wd=rnd(sh.hidden, sh.inter)))
        self.ln_f = torch.ones(sh.hidden, dtype=torch.bfloat16, device=device)
        cache = (sh.layers, S, sh.kv_heads, Lmax, sh.head_dim)
        self.k_cache = torch.zeros(cache, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.zeros(cache, dtype=torch.bfloat16, device=device)
        half = sh.head_dim // 2
        inv = 1.0 / (sh.rope_base ** (torch.arange(0, half, dtype=torch.float64) / half))
        ang = torch.arange(Lmax, dtype=torch.float64)[:, None] * inv[None, :]
        self.cos_h = ang.cos().float().to(device).contiguous()  # [Lmax, D/2]
        self.sin_h = ang.sin().float().to(device).contiguous()
        self.cos = torch.cat([self.cos_h, self.cos_h], 1)  # [Lmax, D]
        self.sin = torch.cat([self.sin_h, self.sin_h], 1)
        self.rows = torch.arange(S, device=device)
        self.scale = 1.0 / math.sqrt(sh.head_dim)
        self._attn_out = torch.empty((S, sh.heads, sh.head_dim), dtype=torch.bfloat16,
                                     device=device)
        from . import decode_attention_rope_workspace_bytes
        self._ws = torch.empty(decode_attention_rope_workspace_bytes(S, sh.heads, sh.kv_heads,
                                                                     Lmax, sh.head_dim),
                               dtype=torch.uint8, device=device)

    def fill_cache(self, seed: int, std: float = 1.0):
        """Random keys and values in every cached position (a stand-in for a
        prompt's prefill when only the decode step is measured)."""
        g = torch.Generator(device=self.device)
        g.manual_seed(seed)
        for c in (self.k_cache, self.v_cache):
            c.copy_((torch.randn(c.shape, generator=g, device=self.device) * std).to(c.dtype))

    def _rms(self, x, w):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + self.shape.eps)
                * w.float()).to(torch.bfloat16)

    def _rope(self, t, cos, sin):
        # t [S, heads, D] bfloat16; rotate-half form in binary32
        tf = t.float()
        h = tf.shape[-1] // 2
        rot = torch.cat([-tf[..., h:], tf[..., :h]], -1)
        return (tf * cos[:, None, :] + rot * sin[:, None, :]).to(torch.bfloat16)

    def _attention_reference(self, q, kc, vc, lens):
        sh = self.shape
        grp = sh.heads // sh.kv_heads
        qf = q.float().view(self.S, sh.kv_heads, grp, sh.head_dim)
        s = torch.einsum("sgqd,sgld->sgql", qf, kc.float()) * self.scale
        valid = torch.arange(self.Lmax, device=self.device)[None, :] < lens[:, None].long()
        s = s.masked_fill(~valid[:, None, None, :], float("-inf"))
        o = torch.einsum("sgql,sgld->sgqd", torch.softmax(s, -1), vc.float())
        return o.reshape(self.S, sh.heads, sh.head_dim).to(torch.bfloat16)

    def step(self, tok: torch.Tensor, pos: torch.Tensor, attention: str = "library"):
        from . import decode_attention, decode_attention_rope
        if attention not in ("library", "library_unfused", "reference"):
            raise ValueError(f"unknown attention {attention!r}")
        sh = self.shape
        nq, nkv = sh.heads * sh.head_dim, sh.kv_heads * sh.head_dim
        S = self.S
        if attention != "library":  # the fused call gathers the angles itself
            cos, sin = self.cos[pos.long()], self.sin[pos.long()]  # [S, D]
            lens = pos + 1
        x = self.embed[tok]  # [S, hidden]
        for li, L in enumerate(self.layers):
            h = self._rms(x, L["ln1"])
            qkv = F.linear(h, L["wqkv"], L["bqkv"])
            kc, vc = self.k_cache[li], self.v_cache[li]
            if attention == "library":
                # rotary embedding, cache append and attention in one library call
                a = decode_attention_rope(qkv, self.cos_h, self.sin_h, pos, kc, vc, sh.heads,
                                          self.scale, workspace=self._ws, out=self._attn_out)
            else:
                q = self._rope(qkv[:, :nq].reshape(S, sh.heads, sh.head_dim), cos, sin)
                k = self._rope(qkv[:, nq:nq + nkv].reshape(S, sh.kv_heads, sh.head_dim), cos, sin)
                v = qkv[:, nq + nkv:].reshape(S, sh.kv_heads, sh.head_dim)
                kc[self.rows, :, pos.long(), :] = k
                vc[self.rows, :, pos.long(), :] = v
                if attention == "library_unfused":
                    a = decode_attention(q.contiguous(), kc, vc, lens, self.scale,
                                         workspace=self._ws, out=self._attn_out)
                else:
                    a = self._attention_reference(q, kc, vc, lens)
            x = x + F.linear(a.reshape(S, nq), L["wo"])
            h = self._rms(x, L["ln2"])
            gu = F.linear(h, L["wgu"])
            x = x + F.linear(F.silu(gu[:, :sh.inter]) * gu[:, sh.inter:], L["wd"])
        logits = F.linear(self._rms(x, self.ln_f), self.embed)
        return logits, torch.argmax(logits, -1)
