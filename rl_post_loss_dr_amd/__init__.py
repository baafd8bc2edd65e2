"""Fused Dr. GRPO update loss (forward + backward) on AMD Instinct MI355X.

Thin Python binding over the C ABI of ``libdrgrpo.so`` (declared in
``include/drgrpo.h``).  This module only checks and marshals arguments:
every step of the loss runs in the library's HIP kernels.  PyTorch provides
device memory and the current stream.  There is no CPU fallback: if the
library is missing, every call raises.

Definitions follow "Making Dr GRPO go brrr" ("The completion mask",
"compute_logprobs", "PPO", "Dr. GRPO", "The loss"); see ``drgrpo.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB, build  # noqa: F401

F32, BF16 = 0, 1

OK = 0
ERR_NULL, ERR_SHAPE, ERR_PARAM, ERR_DTYPE = -1, -2, -3, -4
ERR_WORKSPACE, ERR_ALIGN, ERR_HIP, ERR_TOKEN_RANGE, ERR_ALIAS = -5, -6, -7, -8, -9
ERR_SCRATCH_LIMIT = -10
NOALLOC_SCRATCH_BYTES = 16 << 20  # DRGRPO_NOALLOC_SCRATCH_BYTES


class DrGRPOError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (status {code})")


ADV_CENTER, ADV_ZSCORE = 0, 1                          # Dr. GRPO, GRPO advantages
AGG_TOKEN_SUM, AGG_SEQ_MEAN, AGG_TOKEN_MEAN = 0, 1, 2  # aggregation (drgrpo_agg_mode_t)


class _Variant(ctypes.Structure):
    _fields_ = [("adv_mode", ctypes.c_int32), ("agg_mode", ctypes.c_int32)]


class _Aux(ctypes.Structure):
    _fields_ = [("len", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("adv", ctypes.c_void_p),
                ("logp", ctypes.c_void_p), ("tok_loss", ctypes.c_void_p),
                ("stats", ctypes.c_void_p)]


class _LossOpts(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_void_p), ("token_counts", ctypes.c_void_p),
                ("rows_event_begin", ctypes.c_void_p), ("rows_event_end", ctypes.c_void_p),
                ("require_vector_path", ctypes.c_int32)]


_lib = None
_P, _I64, _F, _SZ, _I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t,
                         ctypes.c_int)


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(
                f"{LIB} is missing: the fused Dr. GRPO loss needs its HIP library "
                "(build it with rl_post_loss_dr_amd.build()); there is no CPU fallback")
        L = ctypes.CDLL(LIB)
        L.drgrpo_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64]
        L.drgrpo_workspace_bytes.restype = _SZ
        common = [_P, _P, _I64, _P, _P, _P, _I64, _F, _F, _F, _P, _P, _I64, _I64, _I64, _I, _P,
                  _SZ, _P]
        L.drgrpo_loss_fwd_bwd.argtypes = common
        L.drgrpo_loss_fwd_bwd.restype = _I
        L.drgrpo_loss_fwd_bwd_ex.argtypes = common + [ctypes.POINTER(_Aux)]
        L.drgrpo_loss_fwd_bwd_ex.restype = _I
        L.drgrpo_loss_fwd_bwd_opts.argtypes = common + [ctypes.POINTER(_Aux),
                                                        ctypes.POINTER(_LossOpts)]
        L.drgrpo_loss_fwd_bwd_opts.restype = _I
        L.drgrpo_loss_fwd_bwd_noalloc.argtypes = common[:16] + [_P]
        L.drgrpo_loss_fwd_bwd_noalloc.restype = _I
        L.drgrpo_completion_mask.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
        L.drgrpo_completion_mask.restype = _I
        L.drgrpo_group_advantage.argtypes = [_P, _I64, _I64, _P, _P, _P]
        L.drgrpo_group_advantage.restype = _I
        L.drgrpo_group_advantage_ex.argtypes = [_P, _I64, _I64, ctypes.c_int32, _P, _P, _P]
        L.drgrpo_group_advantage_ex.restype = _I
        L.drgrpo_logprobs.argtypes = [_P, _P, _I64, _I64, _I64, _I, _P, _P]
        L.drgrpo_logprobs.restype = _I
        L.drgrpo_lmhead_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64]
        L.drgrpo_lmhead_workspace_bytes.restype = _SZ
        L.drgrpo_lmhead_loss_fwd_bwd.argtypes = [_P, _P, _P, _I64, _P, _P, _P, _I64, _F, _F, _F,
                                                 _P, _P, _P, _I64, _I64, _I64, _I64, _P, _SZ, _P]
        L.drgrpo_lmhead_loss_fwd_bwd.restype = _I
        L.drgrpo_lmhead_loss_fwd_bwd_ex.argtypes = L.drgrpo_lmhead_loss_fwd_bwd.argtypes + [
            ctypes.POINTER(_Variant), ctypes.c_void_p]
        L.drgrpo_lmhead_loss_fwd_bwd_ex.restype = _I
        L.drgrpo_lmhead_logprobs_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64]
        L.drgrpo_lmhead_logprobs_workspace_bytes.restype = _SZ
        L.drgrpo_lmhead_logprobs.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P,
                                             _SZ, _P]
        L.drgrpo_lmhead_logprobs.restype = _I
        L.drgrpo_decode_attention_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64]
        L.drgrpo_decode_attention_workspace_bytes.restype = _SZ
        L.drgrpo_decode_attention.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F,
                                              _P, _P, _P, _SZ, _P]
        L.drgrpo_decode_attention.restype = _I
        L.drgrpo_decode_attention_rope_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64]
        L.drgrpo_decode_attention_rope_workspace_bytes.restype = _SZ
        L.drgrpo_decode_attention_rope.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                                   _F, _P, _P, _P, _P, _P, _SZ, _P]
        L.drgrpo_decode_attention_rope.restype = _I
        L.drgrpo_device_status.argtypes = [_P, _P]
        L.drgrpo_device_status.restype = _I
        L.drgrpo_status_string.argtypes = [_I]
        L.drgrpo_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().drgrpo_status_string(code).decode()


def _check(code: int, where: str) -> None:
    if code != OK:
        raise DrGRPOError(code, where)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ws(workspace: torch.Tensor, dev: torch.device) -> torch.Tensor:
    """A caller-supplied workspace: a contiguous uint8 tensor on the inputs'
    device (a host buffer would be written by the kernels)."""
    _dev(workspace, "workspace", torch.uint8)
    if workspace.device != dev:
        raise ValueError(f"workspace must be on {dev}, got {workspace.device}")
    return workspace


def _same_device(dev: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on {dev}, got {t.device}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def workspace_bytes(N: int, C: int, V: int, G: int) -> int:
    return int(lib().drgrpo_workspace_bytes(N, C, V, G))


def make_workspace(N: int, C: int, V: int, G: int, device) -> torch.Tensor:
    n = workspace_bytes(N, C, V, G)
    if n == 0:
        raise DrGRPOError(ERR_SHAPE, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def loss_fwd_bwd(logits: torch.Tensor, tokens: torch.Tensor, eos_id: int, rewards: torch.Tensor,
                 logp_old: torch.Tensor, logp_ref: torch.Tensor | None = None, *, G: int,
                 eps: float = 0.2, beta: float = 0.0, norm_const: float | None = None,
                 out_dlogits: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 aux: dict | None = None, rows_events=None, adv_mode: int = ADV_CENTER,
                 agg: int = AGG_TOKEN_SUM, out_counts: torch.Tensor | None = None,
                 require_vector_path: bool = False):
    """Loss and dlogits of the Dr. GRPO update for one rollout batch.

    logits [N, C, V] float32/bfloat16 (the completion slice: row t scores
    tokens[:, t]); tokens [N, C] int64; rewards [N] float32; logp_old,
    logp_ref [N, C] float32.  norm_const defaults to G*C.  Returns
    (loss [] float32 device tensor, dlogits like logits).  `out_dlogits` may
    be `logits` itself (in place).  `aux` (a dict) receives device tensors
    len, mask, adv, logp, tok_loss and stats (int32 [4]) when given;
    `out_counts` (int64 [2] device tensor) receives the counted and active
    tokens.  `rows_events` is an
    optional pair of recorded torch.cuda.Event (enable_timing=True) that the
    library records around its per-row kernel on the current stream.
    adv_mode / agg select GRPO's normalisations (ADV_ZSCORE, AGG_SEQ_MEAN) or
    the token mean (AGG_TOKEN_MEAN) instead of Dr. GRPO's.
    require_vector_path turns an operand that would take the element path
    (row bytes not a multiple of 16, unaligned bases) into ERR_ALIGN.
    """
    if logits.dim() != 3:
        raise ValueError("logits must be [N, C, V]")
    N, C, V = logits.shape
    dt = _dtype_code(logits)
    _dev(logits, "logits", logits.dtype)
    dev = logits.device
    _dev(tokens, "tokens", torch.int64, (N, C))
    _dev(rewards, "rewards", torch.float32, (N,))
    _dev(logp_old, "logp_old", torch.float32, (N, C))
    if logp_ref is not None:
        _dev(logp_ref, "logp_ref", torch.float32, (N, C))
    if norm_const is None:
        norm_const = float(G * C)
    if out_dlogits is None:
        out_dlogits = torch.empty_like(logits)
    else:
        _dev(out_dlogits, "out_dlogits", logits.dtype, (N, C, V))
    _same_device(dev, tokens=tokens, rewards=rewards, logp_old=logp_old, logp_ref=logp_ref,
                 out_dlogits=out_dlogits)
    if workspace is None:
        workspace = make_workspace(N, C, V, G, dev)
    else:
        _ws(workspace, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    args = (logits.data_ptr(), tokens.data_ptr(), int(eos_id), rewards.data_ptr(),
            logp_old.data_ptr(), _ptr(logp_ref), int(G), float(eps), float(beta),
            float(norm_const), loss.data_ptr(), out_dlogits.data_ptr(), N, C, V, dt,
            workspace.data_ptr(), workspace.numel(), _stream(dev))
    if out_counts is not None:
        _dev(out_counts, "out_counts", torch.int64, (2,))
        _same_device(dev, out_counts=out_counts)
    variant = (adv_mode, agg) != (ADV_CENTER, AGG_TOKEN_SUM)
    opts_needed = (variant or rows_events is not None or require_vector_path or
                   out_counts is not None)
    if aux is None and not opts_needed:
        _check(lib().drgrpo_loss_fwd_bwd(*args), "drgrpo_loss_fwd_bwd")
        return loss, out_dlogits
    s = _Aux()
    if aux is not None:
        aux["len"] = torch.empty(N, dtype=torch.int32, device=dev)
        aux["mask"] = torch.empty((N, C), dtype=torch.uint8, device=dev)
        aux["adv"] = torch.empty(N, dtype=torch.float32, device=dev)
        aux["logp"] = torch.empty((N, C), dtype=torch.float32, device=dev)
        aux["tok_loss"] = torch.empty((N, C), dtype=torch.float32, device=dev)
        aux["stats"] = torch.empty(4, dtype=torch.int32, device=dev)
        for k in ("len", "mask", "adv", "logp", "tok_loss", "stats"):
            setattr(s, k, aux[k].data_ptr())
    if not opts_needed:
        _check(lib().drgrpo_loss_fwd_bwd_ex(*args, ctypes.byref(s)), "drgrpo_loss_fwd_bwd_ex")
        return loss, out_dlogits
    var = _Variant(int(adv_mode), int(agg))
    o = _LossOpts()
    if variant:
        o.variant = ctypes.addressof(var)
    if out_counts is not None:
        o.token_counts = out_counts.data_ptr()
    if rows_events is not None:
        o.rows_event_begin = rows_events[0].cuda_event
        o.rows_event_end = rows_events[1].cuda_event
    o.require_vector_path = 1 if require_vector_path else 0
    _check(lib().drgrpo_loss_fwd_bwd_opts(*args, ctypes.byref(s), ctypes.byref(o)),
           "drgrpo_loss_fwd_bwd_opts")
    return loss, out_dlogits


def loss_fwd_bwd_noalloc(logits: torch.Tensor, tokens: torch.Tensor, eos_id: int,
                         rewards: torch.Tensor, logp_old: torch.Tensor,
                         logp_ref: torch.Tensor | None, *, G: int, eps: float = 0.2,
                         beta: float = 0.0, norm_const: float | None = None,
                         out_loss: torch.Tensor, out_dlogits: torch.Tensor):
    """loss_fwd_bwd through drgrpo_loss_fwd_bwd_noalloc: no workspace, and no
    device memory allocated by this call or the library (the caller passes the
    outputs: out_loss a float32 scalar, out_dlogits like logits).  Returns
    (out_loss, out_dlogits)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [N, C, V]")
    N, C, V = logits.shape
    dt = _dtype_code(logits)
    _dev(logits, "logits", logits.dtype)
    dev = logits.device
    _dev(tokens, "tokens", torch.int64, (N, C))
    _dev(rewards, "rewards", torch.float32, (N,))
    _dev(logp_old, "logp_old", torch.float32, (N, C))
    if logp_ref is not None:
        _dev(logp_ref, "logp_ref", torch.float32, (N, C))
    _dev(out_loss, "out_loss", torch.float32)
    if out_loss.numel() != 1:
        raise ValueError("out_loss must hold one element")
    _dev(out_dlogits, "out_dlogits", logits.dtype, (N, C, V))
    _same_device(dev, tokens=tokens, rewards=rewards, logp_old=logp_old, logp_ref=logp_ref,
                 out_loss=out_loss, out_dlogits=out_dlogits)
    if norm_const is None:
        norm_const = float(G * C)
    _check(lib().drgrpo_loss_fwd_bwd_noalloc(
        logits.data_ptr(), tokens.data_ptr(), int(eos_id), rewards.data_ptr(),
        logp_old.data_ptr(), _ptr(logp_ref), int(G), float(eps), float(beta), float(norm_const),
        out_loss.data_ptr(), out_dlogits.data_ptr(), N, C, V, dt, _stream(dev)),
        "drgrpo_loss_fwd_bwd_noalloc")
    return out_loss, out_dlogits


def logprobs(logits: torch.Tensor, tokens: torch.Tensor) -> torch.Tensor:
    """Forward-only log-probs [N, C] float32 of every token (no mask)."""
    if logits.dim() != 3:
        raise ValueError("logits must be [N, C, V]")
    N, C, V = logits.shape
    dt = _dtype_code(logits)
    _dev(logits, "logits", logits.dtype)
    _dev(tokens, "tokens", torch.int64, (N, C))
    out = torch.empty((N, C), dtype=torch.float32, device=logits.device)
    _check(lib().drgrpo_logprobs(logits.data_ptr(), tokens.data_ptr(), N, C, V, dt,
                                 out.data_ptr(), _stream(logits.device)), "drgrpo_logprobs")
    return out


def completion_mask(tokens: torch.Tensor, eos_id: int):
    """(len int32 [N], mask uint8 [N, C]) of the first-EOS-inclusive mask."""
    _dev(tokens, "tokens", torch.int64)
    N, C = tokens.shape
    ln = torch.empty(N, dtype=torch.int32, device=tokens.device)
    mk = torch.empty((N, C), dtype=torch.uint8, device=tokens.device)
    _check(lib().drgrpo_completion_mask(tokens.data_ptr(), N, C, int(eos_id), ln.data_ptr(),
                                        mk.data_ptr(), _stream(tokens.device)),
           "drgrpo_completion_mask")
    return ln, mk


def group_advantage(rewards: torch.Tensor, G: int, mode: int = ADV_CENTER):
    """(advantages float32 [N], no-contrast group count int32 [1])."""
    _dev(rewards, "rewards", torch.float32)
    N = rewards.numel()
    adv = torch.empty(N, dtype=torch.float32, device=rewards.device)
    cnt = torch.empty(1, dtype=torch.int32, device=rewards.device)
    if mode == ADV_CENTER:
        _check(lib().drgrpo_group_advantage(rewards.data_ptr(), N, int(G), adv.data_ptr(),
                                            cnt.data_ptr(), _stream(rewards.device)),
               "drgrpo_group_advantage")
    else:
        _check(lib().drgrpo_group_advantage_ex(rewards.data_ptr(), N, int(G), int(mode),
                                               adv.data_ptr(), cnt.data_ptr(),
                                               _stream(rewards.device)),
               "drgrpo_group_advantage_ex")
    return adv, cnt


def device_status(workspace: torch.Tensor) -> int:
    """Synchronises the current stream and returns the status word of the last
    loss call that used `workspace` (OK or ERR_TOKEN_RANGE)."""
    _dev(workspace, "workspace", torch.uint8)
    return int(lib().drgrpo_device_status(workspace.data_ptr(), _stream(workspace.device)))


def lmhead_workspace_bytes(N: int, C: int, V: int, H: int, G: int) -> int:
    return int(lib().drgrpo_lmhead_workspace_bytes(N, C, V, H, G))


def lmhead_loss_fwd_bwd(hidden: torch.Tensor, W: torch.Tensor, tokens: torch.Tensor, eos_id: int,
                        rewards: torch.Tensor, logp_old: torch.Tensor,
                        logp_ref: torch.Tensor | None = None, *, G: int, eps: float = 0.2,
                        beta: float = 0.0, norm_const: float | None = None,
                        out_dhidden: torch.Tensor | None = None,
                        out_dW: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, adv_mode: int = ADV_CENTER,
                        agg: int = AGG_TOKEN_SUM, fwd_events=None):
    """Fused lm_head variant: logits = hidden . W^T are never stored.

    hidden [N*C, H] (or [N, C, H]) bfloat16, W [V, H] bfloat16, tokens [N, C]
    int64.  Returns (loss [] float32, dhidden like hidden, dW like W).
    `fwd_events`: optional pair of torch.cuda.Event (enable_timing=True) that
    the library stamps around its forward log-sum-exp product.
    """
    if tokens.dim() != 2:
        raise ValueError("tokens must be [N, C]")
    N, C = tokens.shape
    V, H = W.shape
    _dev(W, "W", torch.bfloat16)
    _dev(hidden, "hidden", torch.bfloat16)
    if hidden.numel() != N * C * H:
        raise ValueError(f"hidden must hold N*C rows of H={H}")
    dev = hidden.device
    _dev(tokens, "tokens", torch.int64)
    _dev(rewards, "rewards", torch.float32, (N,))
    _dev(logp_old, "logp_old", torch.float32, (N, C))
    if logp_ref is not None:
        _dev(logp_ref, "logp_ref", torch.float32, (N, C))
    if norm_const is None:
        norm_const = float(G * C)
    if out_dhidden is None:
        out_dhidden = torch.empty_like(hidden)
    else:
        _dev(out_dhidden, "out_dhidden", torch.bfloat16, hidden.shape)
    if out_dW is None:
        out_dW = torch.empty_like(W)
    else:
        _dev(out_dW, "out_dW", torch.bfloat16, (V, H))
    _same_device(dev, W=W, tokens=tokens, rewards=rewards, logp_old=logp_old, logp_ref=logp_ref,
                 out_dhidden=out_dhidden, out_dW=out_dW)
    if workspace is None:
        n = lmhead_workspace_bytes(N, C, V, H, G)
        if n == 0:
            raise DrGRPOError(ERR_SHAPE, "drgrpo_lmhead_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _ws(workspace, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    var = _Variant(int(adv_mode), int(agg))
    lmaux = None
    if fwd_events is not None:
        lmaux = (ctypes.c_void_p * 2)(fwd_events[0].cuda_event, fwd_events[1].cuda_event)
    _check(lib().drgrpo_lmhead_loss_fwd_bwd_ex(
        hidden.data_ptr(), W.data_ptr(), tokens.data_ptr(), int(eos_id), rewards.data_ptr(),
        logp_old.data_ptr(), _ptr(logp_ref), int(G), float(eps), float(beta), float(norm_const),
        loss.data_ptr(), out_dhidden.data_ptr(), out_dW.data_ptr(), N, C, V, H,
        workspace.data_ptr(), workspace.numel(), _stream(dev), ctypes.byref(var),
        None if lmaux is None else ctypes.cast(lmaux, ctypes.c_void_p)),
        "drgrpo_lmhead_loss_fwd_bwd_ex")
    return loss, out_dhidden, out_dW


def lmhead_logprobs_workspace_bytes(N: int, C: int, V: int, H: int) -> int:
    return int(lib().drgrpo_lmhead_logprobs_workspace_bytes(N, C, V, H))


def lmhead_logprobs(hidden: torch.Tensor, W: torch.Tensor, tokens: torch.Tensor,
                    eos_id: int = -1, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Forward-only log-probs [N, C] float32 through the fused lm_head (logits
    = hidden . W^T never stored): counted tokens get log_softmax(x)[y], positions
    after the first EOS get 0 (eos_id = -1: every token is counted)."""
    if tokens.dim() != 2:
        raise ValueError("tokens must be [N, C]")
    N, C = tokens.shape
    V, H = W.shape
    _dev(W, "W", torch.bfloat16)
    _dev(hidden, "hidden", torch.bfloat16)
    if hidden.numel() != N * C * H:
        raise ValueError(f"hidden must hold N*C rows of H={H}")
    _dev(tokens, "tokens", torch.int64)
    dev = hidden.device
    _same_device(dev, W=W, tokens=tokens)
    if workspace is None:
        n = lmhead_logprobs_workspace_bytes(N, C, V, H)
        if n == 0:
            raise DrGRPOError(ERR_SHAPE, "drgrpo_lmhead_logprobs_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _ws(workspace, dev)
    out = torch.empty((N, C), dtype=torch.float32, device=dev)
    _check(lib().drgrpo_lmhead_logprobs(
        hidden.data_ptr(), W.data_ptr(), tokens.data_ptr(), int(eos_id), N, C, V, H,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)),
        "drgrpo_lmhead_logprobs")
    return out


def decode_attention_workspace_bytes(S: int, Hq: int, Hkv: int, Lmax: int, D: int) -> int:
    return int(lib().drgrpo_decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D))


def decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     lens: torch.Tensor, scale: float | None = None, want_lse: bool = False,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Decode attention of one new token per sequence against its KV cache.

    q [S, Hq, D], k_cache / v_cache [S, Hkv, Lmax, D] bfloat16, lens [S] int32
    (cached positions per sequence).  Returns out [S, Hq, D] bfloat16 (and the
    float32 log-sum-exp [S, Hq] when want_lse).  scale defaults to 1/sqrt(D).
    """
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [S, Hq, D] and the caches [S, Hkv, Lmax, D]")
    S, Hq, D = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    _dev(q, "q", torch.bfloat16)
    _dev(k_cache, "k_cache", torch.bfloat16, (S, Hkv, Lmax, D))
    _dev(v_cache, "v_cache", torch.bfloat16, (S, Hkv, Lmax, D))
    _dev(lens, "lens", torch.int32, (S,))
    dev = q.device
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    _same_device(dev, k_cache=k_cache, v_cache=v_cache, lens=lens)
    if workspace is None:
        n = decode_attention_workspace_bytes(S, Hq, Hkv, Lmax, D)
        if n == 0:
            raise DrGRPOError(ERR_SHAPE, "drgrpo_decode_attention_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _ws(workspace, dev)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    else:
        _dev(out, "out", torch.bfloat16, (S, Hq, D))
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev) if want_lse else None
    _check(lib().drgrpo_decode_attention(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), lens.data_ptr(), S, Hq, Hkv, Lmax,
        D, float(scale), out.data_ptr(), _ptr(lse), workspace.data_ptr(), workspace.numel(),
        _stream(dev)), "drgrpo_decode_attention")
    return (out, lse) if want_lse else out


def decode_attention_rope_workspace_bytes(S: int, Hq: int, Hkv: int, Lmax: int, D: int) -> int:
    return int(lib().drgrpo_decode_attention_rope_workspace_bytes(S, Hq, Hkv, Lmax, D))


def decode_attention_rope(qkv: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                          pos: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, Hq: int,
                          scale: float | None = None, want_lse: bool = False,
                          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """The decode step's attention block: rotary embedding of the new token's
    query and key heads (rotate-half form), append of its key and value to
    the caches at pos, then decode attention over pos + 1 positions.

    qkv [S, (Hq + 2 Hkv) * D] bfloat16 (query, key, value heads), rope_cos /
    rope_sin [Lmax, D/2] float32, pos [S] int32, caches [S, Hkv, Lmax, D]
    bfloat16 (updated in place).  Returns out [S, Hq, D] bfloat16 (and the
    float32 log-sum-exp when want_lse)."""
    S, Hkv, Lmax, D = k_cache.shape
    dev = k_cache.device
    _dev(k_cache, "k_cache", torch.bfloat16)
    _dev(v_cache, "v_cache", torch.bfloat16, (S, Hkv, Lmax, D))
    _dev(qkv, "qkv", torch.bfloat16, (S, (Hq + 2 * Hkv) * D))
    _dev(rope_cos, "rope_cos", torch.float32, (Lmax, D // 2))
    _dev(rope_sin, "rope_sin", torch.float32, (Lmax, D // 2))
    _dev(pos, "pos", torch.int32, (S,))
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    _same_device(dev, qkv=qkv, v_cache=v_cache, rope_cos=rope_cos, rope_sin=rope_sin, pos=pos)
    if workspace is None:
        n = decode_attention_rope_workspace_bytes(S, Hq, Hkv, Lmax, D)
        if n == 0:
            raise DrGRPOError(ERR_SHAPE, "drgrpo_decode_attention_rope_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    else:
        _ws(workspace, dev)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev)
    else:
        _dev(out, "out", torch.bfloat16, (S, Hq, D))
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev) if want_lse else None
    _check(lib().drgrpo_decode_attention_rope(
        qkv.data_ptr(), rope_cos.data_ptr(), rope_sin.data_ptr(), pos.data_ptr(), S, Hq, Hkv,
        Lmax, D, float(scale), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), _ptr(lse),
        workspace.data_ptr(), workspace.numel(), _stream(dev)), "drgrpo_decode_attention_rope")
    return (out, lse) if want_lse else out


class DrGRPOLoss(torch.autograd.Function):
    """Autograd wrapper: forward returns the loss, backward returns
    grad_out * dlogits for the logits (no gradient to any other input)."""

    @staticmethod
    def forward(ctx, logits, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta,
                norm_const):
        loss, dlogits = loss_fwd_bwd(logits.detach(), tokens, eos_id, rewards, logp_old,
                                     logp_ref, G=G, eps=eps, beta=beta, norm_const=norm_const)
        ctx.save_for_backward(dlogits)
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        (dlogits,) = ctx.saved_tensors
        none = (None,) * 9
        # loss.backward() on this loss alone seeds grad_out = 1: dlogits is then
        # the gradient as it stands, and a multiply would stream all of it
        # through HBM again.  Reading the seed syncs the stream, so it is
        # skipped while a graph is being captured.
        if not torch.cuda.is_current_stream_capturing() and float(grad_out) == 1.0:
            return (dlogits,) + none
        return (dlogits * grad_out.to(dlogits.dtype),) + none
