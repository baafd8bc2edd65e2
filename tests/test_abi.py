"""Boundary tests that need no GPU: the C-ABI library loads, exports every
symbol include/drgrpo.h declares, and rejects bad arguments before launching
anything."""
import ctypes
import os
import re

import pytest

import rl_post_loss_dr_amd as dr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "drgrpo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(drgrpo_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dr.LIB):
        dr.build()
    return dr.lib()


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert "drgrpo_loss_fwd_bwd" in names and len(names) >= 8
    for n in names:
        assert hasattr(L, n), n


def test_workspace_bytes(L):
    assert L.drgrpo_workspace_bytes(64, 256, 151936, 8) > 64 * 256 * 8
    assert L.drgrpo_workspace_bytes(0, 256, 151936, 8) == 0
    assert L.drgrpo_workspace_bytes(64, 256, 151936, 7) == 0
    assert L.drgrpo_workspace_bytes(64, 0, 10, 8) == 0


def test_status_strings(L):
    for code in range(-10, 1):
        assert dr.status_string(code)
    assert "unknown" in dr.status_string(-99)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _call(L, **kw):
    a = dict(logits=FAKE, tokens=FAKE, eos=0, rewards=FAKE, old=FAKE, ref=None, G=8, eps=0.2,
             beta=0.0, kappa=2048.0, loss=FAKE, dl=FAKE * 1000000, N=64, C=256, V=151936,
             dtype=1, ws=FAKE * 4096, wsb=1 << 40, stream=None)
    a.update(kw)
    return L.drgrpo_loss_fwd_bwd(a["logits"], a["tokens"], a["eos"], a["rewards"], a["old"],
                                 a["ref"], a["G"], a["eps"], a["beta"], a["kappa"], a["loss"],
                                 a["dl"], a["N"], a["C"], a["V"], a["dtype"], a["ws"], a["wsb"],
                                 a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), dr.ERR_NULL),
    (dict(tokens=None), dr.ERR_NULL),
    (dict(rewards=None), dr.ERR_NULL),
    (dict(old=None), dr.ERR_NULL),
    (dict(loss=None), dr.ERR_NULL),
    (dict(dl=None), dr.ERR_NULL),
    (dict(beta=0.04, ref=None), dr.ERR_NULL),
    (dict(N=0), dr.ERR_SHAPE),
    (dict(C=-1), dr.ERR_SHAPE),
    (dict(V=0), dr.ERR_SHAPE),
    (dict(G=0), dr.ERR_SHAPE),
    (dict(G=7), dr.ERR_SHAPE),
    (dict(N=1 << 40, C=1 << 30), dr.ERR_SHAPE),
    (dict(eps=-0.1), dr.ERR_PARAM),
    (dict(eps=float("nan")), dr.ERR_PARAM),
    (dict(beta=-1.0, ref=FAKE), dr.ERR_PARAM),
    (dict(beta=float("inf"), ref=FAKE), dr.ERR_PARAM),
    (dict(kappa=0.0), dr.ERR_PARAM),
    (dict(kappa=-3.0), dr.ERR_PARAM),
    (dict(kappa=float("inf")), dr.ERR_PARAM),
    (dict(dtype=5), dr.ERR_DTYPE),
    (dict(ws=None), dr.ERR_WORKSPACE),
    (dict(wsb=16), dr.ERR_WORKSPACE),
    (dict(ws=FAKE * 4096 + 8), dr.ERR_WORKSPACE),
    (dict(dl=FAKE + 64), dr.ERR_ALIAS),
])
def test_argument_validation(L, kw, code):
    assert _call(L, **kw) == code


def test_other_entry_points_validate(L):
    assert L.drgrpo_completion_mask(None, 4, 4, 0, FAKE, None, None) == dr.ERR_NULL
    assert L.drgrpo_completion_mask(FAKE, 0, 4, 0, FAKE, None, None) == dr.ERR_SHAPE
    assert L.drgrpo_group_advantage(FAKE, 8, 3, 0, FAKE, None, None) == dr.ERR_SHAPE
    assert L.drgrpo_group_advantage(None, 8, 4, 0, FAKE, None, None) == dr.ERR_NULL
    assert L.drgrpo_group_advantage(FAKE, 8, 4, 2, FAKE, None, None) == dr.ERR_PARAM
    assert L.drgrpo_lmhead_logprobs(None, FAKE, FAKE, 0, 2, 4, 64, 32, FAKE, FAKE, 1 << 30,
                                    None) == dr.ERR_NULL
    assert L.drgrpo_lmhead_logprobs(FAKE, FAKE, FAKE, 0, 2, 4, 64, 30, FAKE, FAKE, 1 << 30,
                                    None) == dr.ERR_SHAPE
    assert L.drgrpo_lmhead_logprobs(FAKE, FAKE, FAKE, 0, 2, 4, 64, 32, FAKE, FAKE, 16,
                                    None) == dr.ERR_WORKSPACE
    assert L.drgrpo_lmhead_logprobs(FAKE + 8, FAKE, FAKE, 0, 2, 4, 64, 32, FAKE, FAKE,
                                    1 << 30, None) == dr.ERR_ALIGN
    assert L.drgrpo_lmhead_logprobs_workspace_bytes(2, 4, 64, 32) > 0
    assert L.drgrpo_decode_attention_workspace_bytes(64, 14, 2, 512, 64) > 0
    assert L.drgrpo_decode_attention_workspace_bytes(64, 14, 3, 512, 64) == 0
    assert L.drgrpo_decode_attention_workspace_bytes(64, 14, 2, 512, 96) == 0
    att = (FAKE, FAKE, FAKE, FAKE, 64, 14, 2, 512, 64, 0.125, FAKE, None, FAKE * 4096, 1 << 30,
           None)
    assert L.drgrpo_decode_attention(None, *att[1:]) == dr.ERR_NULL
    assert L.drgrpo_decode_attention(*att[:5], 15, *att[6:]) == dr.ERR_SHAPE
    assert L.drgrpo_decode_attention(*att[:9], -1.0, *att[10:]) == dr.ERR_PARAM
    assert L.drgrpo_decode_attention(*att[:13], 16, None) == dr.ERR_WORKSPACE
    assert L.drgrpo_decode_attention(FAKE + 8, *att[1:]) == dr.ERR_ALIGN
    assert L.drgrpo_decode_attention(*att[:10], FAKE + 2, *att[11:]) == dr.ERR_ALIGN
    na = L.drgrpo_decode_attention_workspace_bytes(64, 14, 2, 512, 64)
    nr = L.drgrpo_decode_attention_rope_workspace_bytes(64, 14, 2, 512, 64)
    assert nr >= na + 64 * 14 * 64 * 2 + 64 * 4
    assert L.drgrpo_decode_attention_rope_workspace_bytes(64, 14, 3, 512, 64) == 0
    rope = (FAKE, FAKE, FAKE, FAKE, 64, 14, 2, 512, 64, 0.125, FAKE, FAKE, FAKE, None,
            FAKE * 4096, 1 << 30, None)
    assert L.drgrpo_decode_attention_rope(None, *rope[1:]) == dr.ERR_NULL
    assert L.drgrpo_decode_attention_rope(*rope[:3], None, *rope[4:]) == dr.ERR_NULL
    assert L.drgrpo_decode_attention_rope(*rope[:8], 96, *rope[9:]) == dr.ERR_SHAPE
    assert L.drgrpo_decode_attention_rope(*rope[:9], 0.0, *rope[10:]) == dr.ERR_PARAM
    assert L.drgrpo_decode_attention_rope(FAKE + 1, *rope[1:]) == dr.ERR_ALIGN
    assert L.drgrpo_decode_attention_rope(*rope[:10], FAKE + 8, *rope[11:]) == dr.ERR_ALIGN
    assert L.drgrpo_decode_attention_rope(*rope[:15], nr - 1, None) == dr.ERR_WORKSPACE
    assert L.drgrpo_lmhead_logprobs_workspace_bytes(2, 4, 64, 31) == 0
    assert L.drgrpo_logprobs(FAKE, FAKE, 2, 2, 10, 9, FAKE, None) == dr.ERR_DTYPE
    assert L.drgrpo_logprobs(FAKE, FAKE, 2, 0, 10, 1, FAKE, None) == dr.ERR_SHAPE
    assert L.drgrpo_device_status(None, None) == dr.ERR_NULL


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle and has no CPU fallback."""
    pkg = os.path.join(ROOT, "rl_post_loss_dr_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "drgrpo_oracle" not in txt, f


def test_graft_entry_build_compiles_and_imports():
    """The top-level build() entry compiles every native piece in-tree (HIP
    library, generators, oracle) and imports the package."""
    import __graft_entry__

    __graft_entry__.build()
    assert os.path.exists(dr.LIB)


@pytest.mark.parametrize("adv_mode,agg,code", [(0, 0, dr.ERR_WORKSPACE), (1, 2, dr.ERR_WORKSPACE),
                                               (2, 0, dr.ERR_PARAM), (0, 3, dr.ERR_PARAM),
                                               (-1, 0, dr.ERR_PARAM)])
def test_variant_validation(L, adv_mode, agg, code):
    """Unknown normalisation modes are rejected before anything is launched
    (valid ones get as far as the too-small workspace)."""
    var = dr._Variant(adv_mode, agg)
    args = (FAKE, FAKE, 0, FAKE, FAKE, None, 8, 0.2, 0.0, 2048.0, FAKE, FAKE * 1000000, 64, 256,
            151936, 1, FAKE * 4096, 16, None)
    assert L.drgrpo_loss_fwd_bwd_ex(*args, None, ctypes.byref(var)) == code
    lm = (FAKE, FAKE, FAKE, 0, FAKE, FAKE, None, 8, 0.2, 0.0, 2048.0, FAKE, FAKE, FAKE, 64, 256,
          4096, 896, FAKE * 4096, 16, None)
    assert L.drgrpo_lmhead_loss_fwd_bwd_ex(*lm, ctypes.byref(var), None) == code


def test_missing_library_fails_loudly(monkeypatch):
    """Without its HIP library the package raises; it never computes on the CPU."""
    import torch

    monkeypatch.setattr(dr, "LIB", os.path.join(ROOT, "_no_such_dir", "libdrgrpo.so"))
    monkeypatch.setattr(dr, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        dr.lib()
    # host tensors are refused too (no host path to fall back on)
    tokens = torch.zeros((2, 3), dtype=torch.int64)
    with pytest.raises(TypeError, match="device tensor"):
        dr.completion_mask(tokens, 1)


def test_alignment_is_its_own_error(L):
    """A misaligned operand is DRGRPO_ERR_ALIGN, distinct from the overlap
    error, and is reported before anything is launched."""
    lm = [FAKE, FAKE, FAKE, 0, FAKE, FAKE, None, 8, 0.2, 0.0, 2048.0, FAKE, FAKE, FAKE, 64, 256,
          4096, 896, FAKE * 4096, 1 << 40, None]
    for idx in (0, 1, 12, 13):  # hidden, W, out_dhidden, out_dW
        bad = list(lm)
        bad[idx] = FAKE + 8
        assert L.drgrpo_lmhead_loss_fwd_bwd(*bad) == dr.ERR_ALIGN, idx
    assert "alignment" in dr.status_string(dr.ERR_ALIGN)
    assert "overlaps" in dr.status_string(dr.ERR_ALIAS)


def test_noalloc_validates_before_touching_the_scratch(L):
    """The no-allocation entry point returns its host errors (the loss call's,
    then DRGRPO_ERR_SCRATCH_LIMIT for a batch whose workspace exceeds the
    static array) before it looks up the device array or enqueues anything:
    these calls never reach the GPU."""
    base = [FAKE, FAKE, 0, FAKE, FAKE, None, 8, 0.2, 0.0, 2048.0, FAKE, FAKE * 1000000, 64, 256,
            151936, 1, None]

    def call(changes):
        a = list(base)
        for k, v in changes.items():
            a[k] = v
        return L.drgrpo_loss_fwd_bwd_noalloc(*a)

    assert call({0: None}) == dr.ERR_NULL
    assert call({6: 7}) == dr.ERR_SHAPE
    assert call({7: -1.0}) == dr.ERR_PARAM
    assert call({15: 4}) == dr.ERR_DTYPE
    assert call({8: 0.04}) == dr.ERR_NULL  # beta > 0 without logp_ref
    # 2048 x 1024 token rows: a 19 MB workspace, beyond the 12 MiB array
    assert dr.workspace_bytes(2048, 1024, 8, 8) > dr.NOALLOC_SCRATCH_BYTES
    assert call({12: 2048, 13: 1024, 14: 8}) == dr.ERR_SCRATCH_LIMIT
    # the largest batch the header promises fits
    assert dr.workspace_bytes(655360, 1, 151936, 1) <= dr.NOALLOC_SCRATCH_BYTES
    assert dr.workspace_bytes(655360, 1, 8, 1) <= dr.NOALLOC_SCRATCH_BYTES
    # partial overlap of dlogits with logits
    assert call({11: FAKE + 64}) == dr.ERR_ALIAS
