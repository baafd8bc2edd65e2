"""Seeded synthetic inputs of the decode-attention step (one new query token
per sequence against its KV cache).  Holds none of the attention arithmetic:
only the query, key and value tensors and the per-sequence cache lengths.

Shapes follow the Qwen2.5-0.5B-Instruct policy the pages train (14 query
heads sharing 2 key/value heads, head size 64, hidden 896 = 14 * 64) with
B * G sequences decoding together; values are N(0, 1) in bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import BF16, cpu_normal, randint

S_QUERY, S_KEY, S_VALUE, S_KV_LEN = 10, 11, 12, 13


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    S: int          # sequences decoding together (B * G)
    Hq: int         # query heads
    Hkv: int        # key/value heads (Hq % Hkv == 0)
    D: int          # head size
    Lmax: int       # cache capacity per sequence (keys per head)
    ragged: bool = False  # per-sequence lengths uniform in [1, Lmax] (else all Lmax)
    std: float = 1.0
    seed: int = 20261210

    @property
    def scale(self) -> float:
        return 1.0 / float(self.D) ** 0.5


DECODE: dict[str, DecodeConfig] = {}


def _add(c: DecodeConfig) -> DecodeConfig:
    DECODE[c.name] = c
    return c


# The decode step of the rollout batch: B=8 prompts x G=8 completions, a
# 256-token prompt plus 256 generated tokens (the last step of a 256-token
# completion, the bench workload), and a 1024-token cache.
_add(DecodeConfig("decode_s64_l512", S=64, Hq=14, Hkv=2, D=64, Lmax=512))
_add(DecodeConfig("decode_s64_l1024", S=64, Hq=14, Hkv=2, D=64, Lmax=1024))
# a larger rollout batch (B=32 x G=8 sequences), where the cache read is
# bandwidth- rather than latency-bound, and a 512-sequence, 2048-position one
_add(DecodeConfig("decode_s256_l1024", S=256, Hq=14, Hkv=2, D=64, Lmax=1024))
_add(DecodeConfig("decode_s512_l2048", S=512, Hq=14, Hkv=2, D=64, Lmax=2048))
# parity cases: ragged lengths, a tail that is not a multiple of any tile,
# one-key caches, another head geometry
_add(DecodeConfig("decode_ragged", S=9, Hq=14, Hkv=2, D=64, Lmax=333, ragged=True, seed=7101))
_add(DecodeConfig("decode_one_key", S=4, Hq=14, Hkv=2, D=64, Lmax=1, seed=7102))
_add(DecodeConfig("decode_mha_d128", S=3, Hq=4, Hkv=4, D=128, Lmax=200, ragged=True, seed=7103))
_add(DecodeConfig("decode_gqa8", S=5, Hq=16, Hkv=2, D=64, Lmax=1100, ragged=True, seed=7104))
_add(DecodeConfig("decode_gqa16_d128", S=2, Hq=16, Hkv=1, D=128, Lmax=130, ragged=True,
                  seed=7105))
# long caches: more positions per split than one workgroup's loads cover
# (32 splits at most), so a split runs several load groups with the online
# softmax carried across them; ragged lengths leave some splits empty
_add(DecodeConfig("decode_long_d64", S=2, Hq=4, Hkv=1, D=64, Lmax=40000, ragged=True, seed=7106))
_add(DecodeConfig("decode_long_d128", S=2, Hq=4, Hkv=2, D=128, Lmax=20000, ragged=True,
                  seed=7107))


def get_decode_config(name: str) -> DecodeConfig:
    return DECODE[name]


@dataclass
class DecodeCase:
    cfg: DecodeConfig
    q: np.ndarray     # bfloat16 bits [S, Hq, D]
    k: np.ndarray     # bfloat16 bits [S, Hkv, Lmax, D]
    v: np.ndarray     # bfloat16 bits [S, Hkv, Lmax, D]
    lens: np.ndarray  # int32 [S]


def make_decode_case(cfg: DecodeConfig) -> DecodeCase:
    c = cfg
    q = cpu_normal(c.seed, S_QUERY, 0, c.S * c.Hq * c.D, c.std, BF16).reshape(c.S, c.Hq, c.D)
    n = c.S * c.Hkv * c.Lmax * c.D
    k = cpu_normal(c.seed, S_KEY, 0, n, c.std, BF16).reshape(c.S, c.Hkv, c.Lmax, c.D)
    v = cpu_normal(c.seed, S_VALUE, 0, n, c.std, BF16).reshape(c.S, c.Hkv, c.Lmax, c.D)
    if c.ragged:
        lens = (randint(c.seed, S_KV_LEN, np.arange(c.S), c.Lmax) + 1).astype(np.int32)
        lens[0] = c.Lmax
        lens[-1] = 1
    else:
        lens = np.full(c.S, c.Lmax, dtype=np.int32)
    return DecodeCase(cfg=c, q=q, k=k, v=v, lens=lens)
