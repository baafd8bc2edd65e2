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


def test_ceiling_library_exports_and_checks():
    """libceiling.so (the benchmark's measurement kernels) exports every call
    include/ceiling.h declares, and its calls reject bad arguments before
    launching anything."""
    from rl_post_loss_dr_amd.build import CEIL_LIB
    if not os.path.exists(CEIL_LIB):
        dr.build()
    C = ctypes.CDLL(CEIL_LIB)
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ceiling.h")).read(),
                 flags=re.S)
    names = sorted(set(re.findall(r"\b(ceiling_[a-z0-9_]+)\s*\(", src)))
    assert {"ceiling_rows", "ceiling_rows_ticket", "ceiling_device_info"} <= set(names)
    for n in names:
        assert hasattr(C, n), n
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    C.ceiling_rows.argtypes = [P, P, I64, I64, I64, ctypes.c_int32, P, P, P, P, P]
    C.ceiling_rows_ticket.argtypes = [P, P, I64, I64, I64, P, P, I64, P, P, P, P]
    F = 1 << 40
    assert C.ceiling_rows(F, F, 0, 4096, 1, 0, None, None, None, None, None) == -2
    assert C.ceiling_rows(F, F, 8, 4100, 1, 0, None, None, None, None, None) == -2
    assert C.ceiling_rows(F, F, 8, 4096, 1, 7, None, None, None, None, None) == -3
    assert C.ceiling_rows(None, F, 8, 4096, 1, 0, None, None, None, None, None) == -1
    assert C.ceiling_rows(F + 8, F, 8, 4096, 1, 0, None, None, None, None, None) == -6
    ok = [F, F, 8, 4096, 3, F, F, 4, F, None, None, None]
    for idx in (5, 6, 8):  # row_read, class_rows, counters
        bad = list(ok)
        bad[idx] = None
        assert C.ceiling_rows_ticket(*bad) == -1, idx
    for n_read in (-1, 9):
        bad = list(ok)
        bad[7] = n_read
        assert C.ceiling_rows_ticket(*bad) == -2, n_read


def test_workspace_bytes(L):
    assert L.drgrpo_workspace_bytes(64, 256, 151936, 8) > 64 * 256 * 8
    # the dispatch limit: T x 1024 threads below 2^32 (V > 4864)
    assert L.drgrpo_workspace_bytes(1 << 14, 1 << 8, 151936, 8) == 0
    assert L.drgrpo_workspace_bytes((1 << 14) - 8, 1 << 8, 151936, 8) > 0
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
    # one 1024-thread workgroup per token row: at most 2^22 - 1 rows
    (dict(N=1 << 14, C=1 << 8), dr.ERR_SHAPE),
    (dict(N=(1 << 14) - 8, C=1 << 8, ws=None), dr.ERR_WORKSPACE),
    # 256-thread workgroups (V <= 4864): at most 2^24 - 1 rows
    (dict(N=1 << 16, C=1 << 8, V=4864), dr.ERR_SHAPE),
    (dict(N=(1 << 16) - 8, C=1 << 8, V=4864, ws=None), dr.ERR_WORKSPACE),
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
    assert L.drgrpo_group_advantage(FAKE, 8, 3, FAKE, None, None) == dr.ERR_SHAPE
    assert L.drgrpo_group_advantage(None, 8, 4, FAKE, None, None) == dr.ERR_NULL
    assert L.drgrpo_group_advantage_ex(FAKE, 8, 3, 0, FAKE, None, None) == dr.ERR_SHAPE
    assert L.drgrpo_group_advantage_ex(None, 8, 4, 0, FAKE, None, None) == dr.ERR_NULL
    assert L.drgrpo_group_advantage_ex(FAKE, 8, 4, 2, FAKE, None, None) == dr.ERR_PARAM
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
    opts = dr._LossOpts()
    opts.variant = ctypes.addressof(var)
    assert L.drgrpo_loss_fwd_bwd_opts(*args, None, ctypes.byref(opts)) == code
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
    # 2048 x 1024 token rows: a 19 MB workspace, beyond the 16 MiB array
    assert dr.workspace_bytes(2048, 1024, 8, 8) > dr.NOALLOC_SCRATCH_BYTES
    assert call({12: 2048, 13: 1024, 14: 8}) == dr.ERR_SCRATCH_LIMIT
    # the largest batch the header promises fits
    assert dr.workspace_bytes(655360, 1, 151936, 1) <= dr.NOALLOC_SCRATCH_BYTES
    assert dr.workspace_bytes(655360, 1, 8, 1) <= dr.NOALLOC_SCRATCH_BYTES
    # partial overlap of dlogits with logits
    assert call({11: FAKE + 64}) == dr.ERR_ALIAS


# The boundary as built, call by call: the status codes and, for the calls
# the loss's scope names, the parameter types in order (`void* stream` is a
# hipStream_t, so the header needs no HIP include).  Extra calls and options
# (variants, counters, timing hooks, the fused lm_head's variant entry point,
# the decode attention, the no-allocation call) are additions after these.
STATUS = {"DRGRPO_OK": 0, "DRGRPO_ERR_NULL": -1, "DRGRPO_ERR_SHAPE": -2,
          "DRGRPO_ERR_PARAM": -3, "DRGRPO_ERR_DTYPE": -4, "DRGRPO_ERR_WORKSPACE": -5,
          "DRGRPO_ERR_ALIGN": -6, "DRGRPO_ERR_HIP": -7, "DRGRPO_ERR_TOKEN_RANGE": -8,
          "DRGRPO_ERR_ALIAS": -9, "DRGRPO_ERR_SCRATCH_LIMIT": -10}
_LOSS = ("const void*,const int64_t*,int64_t,const float*,const float*,const float*,int64_t,"
         "float,float,float,float*,void*,int64_t,int64_t,int64_t,drgrpo_dtype_t,void*,size_t,"
         "void*")
SIGNATURES = {
    "drgrpo_workspace_bytes": "int64_t,int64_t,int64_t,int64_t",
    "drgrpo_loss_fwd_bwd": _LOSS,
    "drgrpo_loss_fwd_bwd_ex": _LOSS + ",const drgrpo_aux_t*",
    "drgrpo_completion_mask": "const int64_t*,int64_t,int64_t,int64_t,int32_t*,uint8_t*,void*",
    "drgrpo_group_advantage": "const float*,int64_t,int64_t,float*,int32_t*,void*",
    "drgrpo_logprobs": "const void*,const int64_t*,int64_t,int64_t,int64_t,drgrpo_dtype_t,"
                       "float*,void*",
    "drgrpo_lmhead_loss_fwd_bwd": "const void*,const void*,const int64_t*,int64_t,const float*,"
                                  "const float*,const float*,int64_t,float,float,float,float*,"
                                  "void*,void*,int64_t,int64_t,int64_t,int64_t,void*,size_t,void*",
    "drgrpo_device_status": "const void*,void*",
    "drgrpo_status_string": "int",
}
AUX_FIELDS = ["int32_t* len", "uint8_t* mask", "float* adv", "float* logp", "float* tok_loss",
              "int32_t* stats"]


def _header():
    src = open(os.path.join(ROOT, "include", "drgrpo.h")).read()
    return re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def _norm_type(t):
    t = re.sub(r"\s+", " ", t.strip())
    return re.sub(r"\s*\*", "*", t)


def test_boundary_matches_its_record():
    src = _header()
    enum = dict((k, int(v)) for k, v in re.findall(r"\b(DRGRPO_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", src))
    assert enum == STATUS
    decls = {}
    for name, params in re.findall(r"\b(drgrpo_\w+)\s*\(([^;{]*?)\)\s*;", src, flags=re.S):
        types = [_norm_type(re.sub(r"\b\w+\s*$", "", p)) for p in params.split(",")]
        decls[name] = ",".join(types)
    for name, sig in SIGNATURES.items():
        assert decls.get(name) == sig, (name, decls.get(name))
    body = re.search(r"typedef struct drgrpo_aux \{(.*?)\} drgrpo_aux_t;", src, flags=re.S).group(1)
    fields = [_norm_type(f.strip()).replace("*", "* ").replace("  ", " ").strip()
              for f in body.split(";") if f.strip()]
    assert fields == AUX_FIELDS
    # the status codes the binding mirrors
    for k, v in STATUS.items():
        assert getattr(dr, k.replace("DRGRPO_", "")) == v, k


def test_require_vector_path_turns_the_element_path_into_an_align_error(L):
    """Opt-in strict mode: a bfloat16 row whose byte size is not a multiple of
    16 (V % 8 != 0) or an unaligned base is DRGRPO_ERR_ALIGN before any
    launch; without it such rows take the element path."""
    args = [FAKE, FAKE, 0, FAKE, FAKE, None, 8, 0.2, 0.0, 2048.0, FAKE, FAKE * 10 ** 7, 64, 256,
            151937, 1, FAKE * 4096, 1 << 40, None]
    opts = dr._LossOpts()
    opts.require_vector_path = 1
    assert L.drgrpo_loss_fwd_bwd_opts(*args, None, ctypes.byref(opts)) == dr.ERR_ALIGN
    args[14] = 151936
    args[0] = FAKE + 2
    assert L.drgrpo_loss_fwd_bwd_opts(*args, None, ctypes.byref(opts)) == dr.ERR_ALIGN
    # float32 rows of any V are a multiple of 4 bytes: V % 4 != 0 is the element path
    args[0], args[14], args[15] = FAKE, 151937, 0
    assert L.drgrpo_loss_fwd_bwd_opts(*args, None, ctypes.byref(opts)) == dr.ERR_ALIGN
