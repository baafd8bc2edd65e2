"""Synthetic workload definitions for the fused Dr. GRPO loss.

The five named workloads follow the shapes of the pages' setup (a
Qwen2.5-0.5B-Instruct policy: vocabulary 151936, hidden 896, EOS id 151645;
G completions per prompt; completion length C) with synthetic values, since
the pages' data (GSM8K prompts, model weights) is neither present nor needed.
The remaining entries are smaller parity cases with the same structure.

Field meanings
--------------
B, G, C, V      prompts, completions per prompt, completion length, vocabulary
dtype           "f32" or "bf16" element type of the logits
logit_std       standard deviation of the synthetic logits
eos_id          end-of-sequence id (may lie outside [0, V): then no row has EOS)
tok_lo, tok_hi  token ids are uniform over [tok_lo, tok_hi) minus eos_id
eos_rows        exactly this many rows (chosen by seeded permutation) get an EOS
eos_t0_rows     of those, this many have the EOS at t = 0 (one-token answers)
eos_pad         after the first EOS, the rest of the row is EOS padding
extra_eos       rows with EOS also get a second EOS later in the row
reward          "bernoulli" (p), "graded" ({0,.25,.5,.75,1}), "tiny" (group 0
                all 1.0, other groups Bernoulli(p) redrawn until not uniform)
old_noise       logp_old = logp + N(0, old_noise^2)
ref_noise       logp_ref = logp + N(0, ref_noise^2) (None: no reference)
eps, beta       clip range and KL weight
kappa           aggregation constant (None: G * C)
H               hidden size for the fused lm_head workload (None otherwise)
"""
from __future__ import annotations

from dataclasses import dataclass, replace

QWEN_V = 151936
QWEN_EOS = 151645
QWEN_H = 896


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    G: int
    C: int
    V: int
    dtype: str = "bf16"
    logit_std: float = 2.0
    eos_id: int = QWEN_EOS
    tok_lo: int = 0
    tok_hi: int = QWEN_V
    eos_rows: int = 0
    eos_t0_rows: int = 0
    eos_pad: bool = False
    extra_eos: bool = False
    reward: str = "bernoulli"
    p: float = 0.05
    old_noise: float = 0.02
    ref_noise: float | None = None
    eps: float = 0.2
    beta: float = 0.0
    kappa: float | None = None
    seed: int = 20261202
    H: int | None = None
    hidden_std: float = 1.0
    w_std: float = 0.02

    @property
    def N(self) -> int:
        return self.B * self.G

    @property
    def T(self) -> int:
        return self.B * self.G * self.C

    @property
    def norm_const(self) -> float:
        return float(self.kappa if self.kappa is not None else self.G * self.C)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


def _round_half_even(x: float) -> int:
    return int(round(x))


CONFIGS: dict[str, Config] = {}


def _add(c: Config) -> Config:
    CONFIGS[c.name] = c
    return c


# The five named workloads (sizes as stated for this loss).
TINY = _add(Config(
    name="tiny_fp32", B=2, G=4, C=16, V=64, dtype="f32", logit_std=1.0, eos_id=0,
    tok_lo=1, tok_hi=64, eos_rows=5, eos_t0_rows=1, reward="tiny", p=0.5, old_noise=0.05,
    seed=20261202 + 1))
QWEN_C256 = _add(Config(
    name="qwen_b8g8c256", B=8, G=8, C=256, V=QWEN_V, eos_rows=_round_half_even(0.7 * 64),
    p=0.05, old_noise=0.02, seed=20261202 + 2))
QWEN_C512 = _add(Config(
    name="qwen_b8g16c512", B=8, G=16, C=512, V=QWEN_V,
    eos_rows=128 - _round_half_even(0.3 * 128), p=0.05, old_noise=0.05, seed=20261202 + 3))
QWEN_KL = _add(Config(
    name="qwen_kl_b16g8c1024", B=16, G=8, C=1024, V=QWEN_V,
    eos_rows=_round_half_even(0.7 * 128), reward="graded", old_noise=0.02, ref_noise=0.1,
    beta=0.04, seed=20261202 + 4))
LMHEAD = _add(Config(
    name="lmhead_b8g8c512", B=8, G=8, C=512, V=QWEN_V, H=QWEN_H,
    eos_rows=_round_half_even(0.7 * 64), p=0.2, old_noise=0.02, seed=20261202 + 5))

NAMED = ["tiny_fp32", "qwen_b8g8c256", "qwen_b8g16c512", "qwen_kl_b16g8c1024", "lmhead_b8g8c512"]
# Dense mode of the B=8, G=8, C=256 batch: no EOS and Bernoulli(0.5) rewards
# (this seed leaves no group without contrast), so every token row is active
# and carries the full 4V bytes: the raw streaming rate of the row kernel.
QWEN_DENSE = _add(Config(
    name="qwen_dense_b8g8c256", B=8, G=8, C=256, V=QWEN_V, eos_rows=0, p=0.5, old_noise=0.02,
    seed=20261202 + 6))

# Parity-only cases the oracle finishes in seconds: several vocab tiles and a
# ragged tail, every edge the method has.
_add(Config(name="mini_bf16", B=2, G=4, C=24, V=QWEN_V, eos_rows=5, eos_t0_rows=1,
            reward="tiny", p=0.5, old_noise=0.05, seed=7001))
_add(Config(name="mini_kl_bf16", B=2, G=4, C=20, V=QWEN_V, eos_rows=4, reward="graded",
            old_noise=0.05, ref_noise=0.1, beta=0.04, seed=7002))
_add(Config(name="ragged_bf16", B=3, G=2, C=9, V=50008, logit_std=2.0, eos_id=17,
            tok_lo=0, tok_hi=50008, eos_rows=3, eos_pad=True, reward="tiny", p=0.5,
            old_noise=0.05, seed=7003))
_add(Config(name="odd_v_f32", B=2, G=3, C=7, V=61, dtype="f32", logit_std=1.5, eos_id=5,
            tok_lo=0, tok_hi=61, eos_rows=3, eos_t0_rows=1, extra_eos=True, reward="tiny",
            p=0.5, old_noise=0.05, seed=7004))
_add(Config(name="odd_v_bf16", B=2, G=3, C=7, V=1001, dtype="bf16", logit_std=1.5, eos_id=5,
            tok_lo=0, tok_hi=1001, eos_rows=3, eos_t0_rows=1, extra_eos=True, reward="tiny",
            p=0.5, old_noise=0.05, seed=7005))
_add(Config(name="clip_heavy_f32", B=2, G=4, C=16, V=200, dtype="f32", logit_std=1.0,
            eos_id=0, tok_lo=1, tok_hi=200, eos_rows=4, reward="graded", old_noise=0.3,
            seed=7006))
_add(Config(name="clip_heavy_bf16", B=2, G=4, C=16, V=4096, logit_std=2.0, eos_id=3,
            tok_lo=0, tok_hi=4096, eos_rows=4, reward="graded", old_noise=0.3, ref_noise=0.2,
            beta=0.04, seed=7007))
_add(Config(name="big_v_f32", B=2, G=2, C=3, V=200003, dtype="f32", logit_std=2.0,
            eos_id=QWEN_EOS, tok_lo=0, tok_hi=200003, eos_rows=2, reward="tiny", p=0.5,
            old_noise=0.05, seed=7008))
_add(Config(name="big_v_bf16", B=2, G=2, C=3, V=262144, logit_std=2.0, eos_id=QWEN_EOS,
            tok_lo=0, tok_hi=262144, eos_rows=2, reward="tiny", p=0.5, old_noise=0.05,
            seed=7009))
# the ticket order's other two row paths: 16-byte binary32 chunks (256 KB rows)
# and 2-byte bfloat16 elements (an odd vocabulary of 98,305 entries)
_add(Config(name="ticket_v4_f32", B=2, G=3, C=4, V=65536, dtype="f32", logit_std=2.0, eos_id=5,
            tok_lo=0, tok_hi=65536, eos_rows=3, eos_t0_rows=1, reward="tiny", p=0.5,
            old_noise=0.05, seed=7018))
_add(Config(name="ticket_odd_bf16", B=2, G=3, C=4, V=98305, logit_std=2.0, eos_id=5,
            tok_lo=0, tok_hi=98305, eos_rows=3, eos_t0_rows=1, reward="tiny", p=0.5,
            old_noise=0.05, ref_noise=0.1, beta=0.04, seed=7019))
# the row kernel's ticket order (rows of 192 KB: V = 98,304 in bfloat16) at
# many completions: 320 completions (the row search's multi-round path) and
# 4104 one-token completions (three rounds), groups with and without contrast
_add(Config(name="many_seq_bf16", B=40, G=8, C=3, V=98304, logit_std=2.0, eos_id=3, tok_lo=0,
            tok_hi=98304, eos_rows=200, eos_t0_rows=40, p=0.15, old_noise=0.05, seed=7015))
_add(Config(name="many_seq_c1_bf16", B=513, G=8, C=1, V=98304, logit_std=2.0, eos_id=3,
            tok_lo=0, tok_hi=98304, eos_rows=400, p=0.1, old_noise=0.05, seed=7016))
_add(Config(name="no_eos_id", B=2, G=2, C=5, V=640, logit_std=1.0, eos_id=-1, tok_lo=0,
            tok_hi=640, eos_rows=0, reward="tiny", p=0.5, old_noise=0.05, seed=7010))
_add(Config(name="lmhead_mini", B=2, G=4, C=32, V=4096, H=QWEN_H, eos_id=3, tok_lo=0,
            tok_hi=4096, eos_rows=5, eos_t0_rows=1, p=0.5, reward="tiny", old_noise=0.02,
            seed=7011))
# two backward vocabulary chunks, a ragged last column tile, a KL term
_add(Config(name="lmhead_multi", B=2, G=2, C=7, V=20488, H=96, eos_id=3, tok_lo=0,
            tok_hi=20488, eos_rows=2, reward="tiny", p=0.5, old_noise=0.05, ref_noise=0.1,
            beta=0.04, w_std=0.1, seed=7012))
# three backward vocabulary chunks (the last ragged), small enough for the
# oracle's full gradients
_add(Config(name="lmhead_chunks3", B=2, G=2, C=4, V=70000, H=64, eos_id=3, tok_lo=0,
            tok_hi=70000, eos_rows=1, reward="tiny", p=0.5, old_noise=0.05, w_std=0.1,
            seed=7014))
# a wide hidden size (Qwen2.5-7B's 3584: 112 reduction steps in the forward
# and dhidden products) with a ragged last column tile
_add(Config(name="lmhead_wide_h", B=2, G=2, C=16, V=8200, H=3584, eos_id=3, tok_lo=0,
            tok_hi=8200, eos_rows=2, eos_t0_rows=1, reward="tiny", p=0.5, old_noise=0.05,
            seed=7017))
# a hidden size that leaves the last 224-column gradient tile partly filled
# (1536 = 6 x 224 + 192: its second wavefront column stores 80 of 112 columns)
_add(Config(name="lmhead_h1536", B=2, G=2, C=12, V=5000, H=1536, eos_id=3, tok_lo=0,
            tok_hi=5000, eos_rows=2, reward="tiny", p=0.5, old_noise=0.05, ref_noise=0.1,
            beta=0.04, seed=7020))
# tiny fp64-checkable shape for finite differences of the lm_head oracle
_add(Config(name="lmhead_fd", B=2, G=2, C=3, V=48, H=32, eos_id=3, tok_lo=0, tok_hi=48,
            eos_rows=1, reward="tiny", p=0.5, old_noise=0.3, ref_noise=0.2, beta=0.04,
            w_std=0.3, seed=7013))


def get_config(name: str) -> Config:
    return CONFIGS[name]
