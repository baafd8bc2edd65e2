"""Benchmark of the fused Dr. GRPO loss forward + backward on one MI355X.

One step = one drgrpo_loss_fwd_bwd call (completion mask, group advantage,
log-prob sweep over the vocabulary, clipped surrogate, token sum, dlogits)
over one synthetic rollout batch resident in HBM.  Prints ONE JSON line.

Default workload: B=8 prompts x G=8 completions x C=256 tokens over the
151,936-entry vocabulary in bfloat16 (the Qwen2.5-0.5B-Instruct-shaped
batch), synthetic seeded inputs.  logp_old is the library's own forward
log-prob plus N(0, 0.02^2) noise, as an update step would receive it.  The
same line carries, under "workloads", the larger loss batches (B=8 G=16
C=512; B=16 G=8 C=1024 with the KL term; the all-active dense batch) and the
fused lm_head (B=8 G=8 C=512, H=896), each timed over several calls in this
process (median and spread), and "ceilings": the row kernel's own access
pattern with no arithmetic (copy, fill, read, and the batch's active / zero
row mix) on the same buffers.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--headline-only] [--no-eager]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "loss fwd+bwd completion tokens/s and HBM GB/s (% of peak), V=151936 bf16"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD published peak


def _alg_bytes(cfg, adv, lens):
    """Algorithmic HBM bytes of the per-row kernel for this batch: an active
    token row reads and writes V elements plus its token id, logp_old (and
    logp_ref); an inactive row writes V zeros and reads its token id."""
    import numpy as np

    esz = 2 if cfg.dtype == "bf16" else 4
    mask = np.arange(cfg.C)[None, :] < lens[:, None]
    active = mask & ((adv[:, None] != 0) | (cfg.beta != 0))
    n_act = int(active.sum())
    n_inact = cfg.T - n_act
    per_act = 2 * esz * cfg.V + 8 + 4 + (4 if cfg.beta != 0 else 0)
    per_inact = esz * cfg.V + 8
    return n_act, n_inact, n_act * per_act + n_inact * per_inact, per_act, per_inact


def _src_hash():
    """Identity of the row kernel's code: sha256[:16] of drgrpo.hip and
    common.h with their comments removed and whitespace collapsed, so an edit
    of comments alone keeps a counter measurement valid."""
    h = hashlib.sha256()
    for p in ("rl_post_loss_dr_amd/csrc/drgrpo.hip", "rl_post_loss_dr_amd/csrc/common.h"):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def _traffic(workload):
    """HBM bytes per launch of the row kernel measured by rocprofv3 counters
    (profiles/), if the committed measurement was taken on the current kernel
    source."""
    p = os.path.join(ROOT, "profiles", f"k_rows_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("src_hash") != _src_hash():
        return None
    return rec.get("bytes_per_launch")


def _row_stride(T: int) -> int:
    """The row kernel's workgroup-to-row stride (coprime with T, near T/phi^2)."""
    import math

    s = int(T * 0.3819660112501051) | 1
    while math.gcd(s, T) != 1:
        s += 1
    return s


_ceil = None


def _ceil_lib():
    """libceiling.so: the measurement kernels and device properties."""
    global _ceil
    if _ceil is None:
        import ctypes

        from rl_post_loss_dr_amd.build import CEIL_LIB

        L = ctypes.CDLL(CEIL_LIB)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.ceiling_rows.argtypes = [P, P, I64, I64, I64, ctypes.c_int32, P, P, P, P, P]
        L.ceiling_rows.restype = ctypes.c_int
        L.ceiling_rows_ticket.argtypes = [P, P, I64, I64, I64, P, P, I64, P, P, P, P]
        L.ceiling_rows_ticket.restype = ctypes.c_int
        L.ceiling_device_info.restype = ctypes.c_int
        _ceil = L
    return _ceil


def provenance(seed):
    """Versions and configuration this measurement ran with."""
    import ctypes
    import platform
    import subprocess

    import torch

    class Info(ctypes.Structure):
        _fields_ = [("name", ctypes.c_char * 256), ("arch", ctypes.c_char * 256),
                    ("compute_units", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                    ("memory_clock_khz", ctypes.c_int32), ("memory_bus_bits", ctypes.c_int32),
                    ("total_mem_bytes", ctypes.c_int64), ("l2_bytes", ctypes.c_int32),
                    ("runtime_version", ctypes.c_int32), ("driver_version", ctypes.c_int32)]

    out = {"seed": seed, "torch": torch.__version__, "torch_hip": torch.version.hip,
           "python": platform.python_version()}
    info = Info()
    if _ceil_lib().ceiling_device_info(0, ctypes.byref(info)) == 0:
        out["device"] = {"name": info.name.decode(), "arch": info.arch.decode(),
                         "compute_units": info.compute_units,
                         "max_clock_mhz": info.clock_khz / 1000.0,
                         "memory_clock_mhz": info.memory_clock_khz / 1000.0,
                         "memory_bus_bits": info.memory_bus_bits,
                         "hbm_gib": round(info.total_mem_bytes / 2 ** 30, 1),
                         "l2_bytes": info.l2_bytes, "hip_runtime_version": info.runtime_version,
                         "driver_version": info.driver_version}
    try:
        with open("/opt/rocm/.info/version") as f:
            out["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        r = subprocess.run(["hipcc", "--version"], capture_output=True, text=True, timeout=30)
        out["hipcc"] = " | ".join(l.strip() for l in r.stdout.splitlines()[:2])
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=30)
        if r.returncode == 0:
            out["git_head"] = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    out["build_flags"] = " ".join(__import__("rl_post_loss_dr_amd.build",
                                             fromlist=["HIPCC_FLAGS"]).HIPCC_FLAGS)
    return out


def host_info():
    host = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            lines = f.read().splitlines()
        kv = {}
        for l in lines:
            if ":" in l:
                k, v = l.split(":", 1)
                kv.setdefault(k.strip(), v.strip())
        host["cpu_model"] = kv.get("model name")
        host["cpu_family_model_stepping"] = "/".join(
            kv.get(k, "?") for k in ("cpu family", "model", "stepping"))
        host["cpu_vendor"] = kv.get("vendor_id")
        host["cpu_mhz"] = kv.get("cpu MHz")
        with open("/proc/meminfo") as f:
            host["ram_gb"] = round(int(next(l for l in f if l.startswith("MemTotal")).split()[1])
                                   / 2 ** 20, 1)
    except (OSError, StopIteration, ValueError):
        pass
    return host


def cpu_baseline(cfg, case, target_s: float = 15.0):
    """The CPU oracle, as it stands, on a strided sample of the workload's token
    rows (whole rows, every group represented)."""
    import numpy as np

    import oracle

    T = cfg.T
    n_rows = 256
    step = max(1, T // n_rows)
    rows = np.arange(0, T, step)[:n_rows]
    tok = case.tokens.reshape(-1)[rows]
    x = case.logits_rows(rows)
    # inputs of the sample (not timed): logp_old from the oracle's own log-probs
    _, lp, _ = oracle.row_logprob(x, tok)
    old = synth_perturb(lp, case.old_noise.reshape(-1)[rows])
    ref = None if case.ref_noise is None else synth_perturb(lp, case.ref_noise.reshape(-1)[rows])
    lens = oracle.completion_len(case.tokens, cfg.eos_id)
    adv_all = oracle.group_advantage(case.rewards, cfg.G)
    i_idx = rows // cfg.C
    t_idx = rows % cfg.C
    adv_s = adv_all[i_idx]
    # each sampled token is its own length-1 "completion" carrying its mask
    lens_s = (t_idx < lens[i_idx]).astype(np.int32)
    eps, beta, kappa = (float(np.float32(v)) for v in (cfg.eps, cfg.beta, cfg.norm_const))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.completion_len(case.tokens, cfg.eos_id)
        oracle.group_advantage(case.rewards, cfg.G)
        lse, logp, _ = oracle.row_logprob(x, tok)
        lam, coef, _ = oracle.token_terms(logp[:, None], old[:, None],
                                          None if ref is None else ref[:, None], adv_s, lens_s,
                                          eps, beta, kappa)
        oracle.loss_sum(lam, kappa)
        oracle.dlogits_rows(x, tok, lse, coef.reshape(-1))
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            break
    tok_s = reps * len(rows) / el
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # the same oracle on one thread (OpenMP's thread count set through its
    # runtime) on the first 16 rows of the sample
    single = None
    try:
        import ctypes

        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        try:
            x1, tok1 = x[:16], tok[:16]
            n1 = 0
            t1 = time.perf_counter()
            while time.perf_counter() - t1 < 3.0:
                l1, lp1, _ = oracle.row_logprob(x1, tok1)
                lam1, coef1, _ = oracle.token_terms(lp1[:, None], old[:16, None], None if ref is None
                                                    else ref[:16, None], adv_s[:16], lens_s[:16],
                                                    eps, beta, kappa)
                oracle.dlogits_rows(x1, tok1, l1, coef1.reshape(-1))
                n1 += 1
            single = {"value": n1 * 16 / (time.perf_counter() - t1), "cores": 1,
                      "sample": f"16 token rows x V={cfg.V}, {n1} passes"}
        finally:
            gomp.omp_set_num_threads(threads)
    except OSError:
        pass
    host = host_info()
    return {"value": tok_s, "unit": "completion tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} token rows (every {step}th of {T}) x V={cfg.V}, "
                      f"{reps} passes in {el:.1f} s; mask and advantage over the whole batch",
            "single_thread": single, "host": host}


def _eager_terms(lp, tokens, eos_id, rewards, logp_old, logp_ref, G, eps, beta, kappa):
    """The method's per-token terms in plain PyTorch from already computed
    log-probs: mask through the first EOS, group-centred advantage, clipped
    min-surrogate, optional k3 KL, token sum over the constant kappa."""
    import torch

    N, C = tokens.shape
    is_eos = tokens == eos_id
    first = torch.where(is_eos.any(1), is_eos.int().argmax(1), torch.full_like(tokens[:, 0], C))
    mask = torch.arange(C, device=tokens.device)[None, :] <= first[:, None]
    grp = rewards.view(-1, G)
    adv = (grp - grp.mean(1, keepdim=True)).reshape(N, 1)
    ratio = torch.exp(lp - logp_old)
    surr = torch.minimum(ratio * adv, torch.clamp(ratio, 1 - eps, 1 + eps) * adv)
    lam = -surr
    if beta != 0.0:
        d = logp_ref - lp
        lam = lam + beta * (torch.exp(d) - d - 1)
    return torch.where(mask, lam, torch.zeros_like(lam)).sum() / kappa


def _time_eager(fn, reps=3):
    """Median of `reps` timed calls of fn() after one untimed call."""
    import numpy as np
    import torch

    fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return float(np.median(ms)), ms


def eager_loss(cfg, logits, tokens, rewards, old, ref, loss_ours, dlogits_ours):
    """The same loss written the plain way in eager PyTorch on the same GPU and
    inputs (log-softmax over V in float32, gather, autograd for dlogits), as
    context for the fused call: its time, and its agreement with the fused
    result."""
    import torch

    torch.cuda.reset_peak_memory_stats()

    def step():
        x = logits.detach().requires_grad_(True)
        lp = torch.log_softmax(x.float(), dim=-1).gather(-1, tokens.unsqueeze(-1)).squeeze(-1)
        loss = _eager_terms(lp, tokens, cfg.eos_id, rewards, old, ref, cfg.G, cfg.eps, cfg.beta,
                            cfg.norm_const)
        loss.backward()
        return loss.detach(), x.grad

    loss, grad = step()
    gmax = float(dlogits_ours.float().abs().max().item())
    diff = float((grad.float() - dlogits_ours.float()).abs().max().item())
    lo = float(loss.item())
    del loss, grad
    med, ms = _time_eager(lambda: step())
    peak = torch.cuda.max_memory_allocated() / 2 ** 30
    torch.cuda.empty_cache()
    return {"what": "the loss and dlogits written the plain way in eager PyTorch on the same "
                    "inputs: float32 log-softmax over V, gather, clipped min-surrogate, token "
                    "sum, autograd for dlogits",
            "ms": med, "ms_all": ms, "speedup_of_fused_call": None,
            "loss": lo, "loss_rel_diff": abs(lo - loss_ours) / max(abs(loss_ours), 1e-30),
            "dlogits_max_abs_diff": diff, "dlogits_max_abs": gmax,
            "peak_allocated_gib": round(peak, 1)}


def eager_lmhead(cfg, hidden, W, tokens, rewards, old, loss_ours, dh_ours, dW_ours):
    """The fused lm_head loss written the plain way in eager PyTorch on the same
    GPU and inputs: the [T, V] logits materialised by a bf16 GEMM, float32
    log-softmax, gather, autograd for dhidden and dW (context for the fused
    call)."""
    import torch

    torch.cuda.reset_peak_memory_stats()
    N, C = tokens.shape

    def step():
        h = hidden.detach().requires_grad_(True)
        w = W.detach().requires_grad_(True)
        logits = torch.nn.functional.linear(h, w)
        lp = torch.log_softmax(logits.float(), dim=-1).gather(
            -1, tokens.reshape(-1, 1)).reshape(N, C)
        loss = _eager_terms(lp, tokens, cfg.eos_id, rewards, old, None, cfg.G, cfg.eps,
                            cfg.beta, cfg.norm_const)
        loss.backward()
        return loss.detach(), h.grad, w.grad

    loss, gh, gw = step()
    rel = lambda a, b: float((a.float() - b.float()).abs().max().item()) / max(
        float(b.float().abs().max().item()), 1e-30)
    lo = float(loss.item())
    res = {"dhidden_max_abs_diff_rel": rel(gh, dh_ours), "dW_max_abs_diff_rel": rel(gw, dW_ours)}
    del loss, gh, gw
    med, ms = _time_eager(lambda: step())
    peak = torch.cuda.max_memory_allocated() / 2 ** 30
    torch.cuda.empty_cache()
    return {"what": "the loss, dhidden and dW written the plain way in eager PyTorch on the same "
                    "inputs: [T, V] logits from a bf16 GEMM over all token rows, float32 "
                    "log-softmax, gather, clipped min-surrogate, token sum, autograd",
            "ms": med, "ms_all": ms, "speedup_of_fused_call": None, "loss": lo,
            "loss_rel_diff": abs(lo - loss_ours) / max(abs(loss_ours), 1e-30), **res,
            "peak_allocated_gib": round(peak, 1)}


def _timed_calls(fn, n=5):
    """Median and spread of n calls of fn() after one untimed call, timed by
    events recorded between the calls on the current stream."""
    import torch

    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    for k in range(n):
        ev[k].record()
        fn()
    ev[n].record()
    torch.cuda.synchronize()
    return _spread([ev[k].elapsed_time(ev[k + 1]) for k in range(n)])


def _spread(xs):
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()), "max": float(a.max()),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def measure_lmhead(cfg, case, steps, warmup, eager=False):
    """Fused lm_head workload: hidden [T, H] and W [V, H] in, loss, dhidden,
    dW out.  Per call: whole-call time (events between calls) and the
    forward product's time (events stamped by its dispatch); with eager, the
    plain PyTorch formulation on the same inputs (context)."""
    import numpy as np
    import torch

    import synth
    import rl_post_loss_dr_amd as dr

    dev = torch.device("cuda:0")
    hidden = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    W = torch.empty((cfg.V, cfg.H), dtype=torch.bfloat16, device=dev)
    synth.gpu_normal_fill(hidden, cfg.seed, synth.S_HIDDEN, 0, cfg.hidden_std)
    synth.gpu_normal_fill(W, cfg.seed, synth.S_WEIGHT, 0, cfg.w_std)
    tokens = torch.from_numpy(case.tokens).to(dev)
    rewards = torch.from_numpy(case.rewards).to(dev)
    # logp_old: the policy's own log-probs from the forward-only fused pass
    # (outside the timed region)
    lp = dr.lmhead_logprobs(hidden, W, tokens, cfg.eos_id).double().cpu().numpy()
    old = torch.from_numpy(synth.perturb(lp, case.old_noise)).to(dev)
    dh = torch.empty_like(hidden)
    dW = torch.empty_like(W)
    ws = torch.empty(dr.lmhead_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H, cfg.G),
                     dtype=torch.uint8, device=dev)
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const, out_dhidden=dh,
              out_dW=dW, workspace=ws)
    _, mask_rows = dr.completion_mask(tokens, cfg.eos_id)
    adv, _ = dr.group_advantage(rewards, cfg.G)
    n_act = int(((mask_rows != 0) & (adv[:, None] != 0)).sum().item())
    for _ in range(warmup):
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, old, None, **kw)
    torch.cuda.synchronize()
    # forward-product events on the stream the library launches on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for k in range(steps):
        cev[k].record()
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, old, None,
                               fwd_events=evs[k], **kw)
    cev[steps].record()
    torch.cuda.synchronize()
    ms_total = cev[0].elapsed_time(cev[steps])
    call_ms = [cev[k].elapsed_time(cev[k + 1]) for k in range(steps)]
    fwd_ms = [a.elapsed_time(b) for a, b in evs]
    per_gemm = 2.0 * n_act * cfg.V * cfg.H  # one product over the active tokens
    executed = _lmhead_executed_flops(n_act, cfg.V, cfg.H)
    med = float(np.median(call_ms))
    fwd_med = float(np.median(fwd_ms))
    req = 3 * per_gemm / (med / 1e3) / 1e12
    # the forward-only fused log-prob pass (old / reference log-probs): one
    # product over every counted token, its logits never stored
    n_cnt = int((mask_rows != 0).sum().item())
    ws_lp = torch.empty(dr.lmhead_logprobs_workspace_bytes(cfg.N, cfg.C, cfg.V, cfg.H),
                        dtype=torch.uint8, device=dev)
    lp_ms = _timed_calls(lambda: dr.lmhead_logprobs(hidden, W, tokens, cfg.eos_id,
                                                    workspace=ws_lp))
    lp_flop = 2.0 * n_cnt * cfg.V * cfg.H
    logprobs_rec = {"entry_point": "drgrpo_lmhead_logprobs", "counted_tokens": n_cnt,
                    "ms": lp_ms, "tflop": lp_flop / 1e12,
                    "tflops": lp_flop / (lp_ms["median"] / 1e3) / 1e12,
                    "frac": lp_flop / (lp_ms["median"] / 1e3) / 1e12 / 2500.0}
    del ws_lp
    eager_rec = None
    if eager:
        loss_t, _, _ = dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, old, None,
                                              **kw)
        eager_rec = eager_lmhead(cfg, hidden, W, tokens, rewards, old, float(loss_t.item()), dh,
                                 dW)
        eager_rec["speedup_of_fused_call"] = eager_rec["ms"] / med
    del kw, hidden, W, dh, dW, ws
    torch.cuda.empty_cache()
    return {
        "workload": cfg.name, "B": cfg.B, "G": cfg.G, "C": cfg.C, "V": cfg.V, "H": cfg.H,
        "token_rows": cfg.T, "active_tokens": n_act, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_total / steps, "call_ms": _spread(call_ms),
        "tokens_per_s": cfg.T / (ms_total / steps / 1e3),
        "forward_product": {"kernel": "k_gemm<GM_LSE>", "ms": _spread(fwd_ms),
                            "tflops": per_gemm / (fwd_med / 1e3) / 1e12,
                            "frac": per_gemm / (fwd_med / 1e3) / 1e12 / 2500.0},
        "required_tflop_per_call": 3 * per_gemm / 1e12,
        "call_tflops_required": req, "call_frac_required": req / 2500.0,
        "call_tflops_executed": executed / (med / 1e3) / 1e12,
        "note": "required = logits, dhidden and dW products over the active tokens; executed "
                "adds the MFMA work of padded tiles (256 x 256 forward tiles, 256 x 224 "
                "gradient tiles); frac against 2.5 PFLOP/s dense bf16",
        "logprobs_pass": logprobs_rec,
        **({"torch_eager": eager_rec} if eager_rec else {}),
    }


def _lmhead_executed_flops(n_act, V, H, tile=256, grad_cols=224, kpad=32, chunk=32768):
    """MFMA work of one fused lm_head call as launched: the forward product
    over all V columns on whole 256 x 256 tiles, the dhidden product (reducing
    over V rounded up to 32) and, per vocabulary chunk, the dW product
    (reducing over the active tokens, padded to 32) on whole 256 x 224 tiles.
    The dhidden term is summed per chunk: the chunks are multiples of 32, so
    the sum equals the one product over V rounded up to 32."""
    ru = lambda x, m: (x + m - 1) // m * m
    f = 2.0 * ru(n_act, tile) * ru(V, tile) * H
    for v0 in range(0, V, chunk):
        wv = min(chunk, V - v0)
        f += 2.0 * ru(n_act, tile) * ru(H, grad_cols) * ru(wv, kpad)
        f += 2.0 * ru(wv, tile) * ru(H, grad_cols) * ru(n_act, kpad)
    return f


def _timed_ceiling(mode, src, dst, rows, row_bytes, stride, row_read, sink, reps=5,
                   ticket=None):
    """Median device time (HIP events stamped by the dispatch) of one
    measurement-kernel launch on the current stream; ticket = (class_rows,
    n_read, counters) for the ticket order."""
    import numpy as np
    import torch

    L = _ceil_lib()
    st = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps + 1)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    for e0, e1 in evs:  # the first launch is a warm-up
        if ticket is None:
            rc = L.ceiling_rows(ptr(src), ptr(dst), rows, row_bytes, stride, mode, ptr(row_read),
                                ptr(sink), st, e0.cuda_event, e1.cuda_event)
        else:
            rc = L.ceiling_rows_ticket(ptr(src), ptr(dst), rows, row_bytes, stride,
                                       ptr(row_read), ptr(ticket[0]), ticket[1], ptr(ticket[2]),
                                       st, e0.cuda_event, e1.cuda_event)
        if rc != 0:
            raise RuntimeError(f"ceiling_rows({mode}) returned {rc}")
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs[1:]]))


def measure_loss(cfg, case, steps, warmup, ceilings=False, eager=False):
    """One loss workload: K timed calls after W warm-up calls; per call the
    whole call (events between calls) and the row kernel (events stamped by
    its dispatch).  With ceilings, the measurement kernels run afterwards on
    the same buffers; with eager, the plain PyTorch formulation on the same
    inputs (context, not the measurement)."""
    import numpy as np
    import torch

    import synth
    import rl_post_loss_dr_amd as dr

    dev = torch.device("cuda:0")
    torch_dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    logits = torch.empty((cfg.N, cfg.C, cfg.V), dtype=torch_dt, device=dev)
    synth.gpu_normal_fill(logits, cfg.seed, synth.S_LOGITS, 0, cfg.logit_std)
    tokens = torch.from_numpy(case.tokens).to(dev)
    rewards = torch.from_numpy(case.rewards).to(dev)
    lp = dr.logprobs(logits, tokens).double().cpu().numpy()
    old = torch.from_numpy(synth.perturb(lp, case.old_noise)).to(dev)
    ref = None if case.ref_noise is None else torch.from_numpy(
        synth.perturb(lp, case.ref_noise)).to(dev)
    dlogits = torch.empty_like(logits)
    ws = dr.make_workspace(cfg.N, cfg.C, cfg.V, cfg.G, dev)
    kw = dict(G=cfg.G, eps=cfg.eps, beta=cfg.beta, norm_const=cfg.norm_const,
              out_dlogits=dlogits, workspace=ws)
    aux = {}
    counts = torch.empty(2, dtype=torch.int64, device=dev)
    dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, aux=aux, out_counts=counts,
                    **kw)
    torch.cuda.synchronize()
    lens = aux["len"].cpu().numpy()
    adv = aux["adv"].cpu().numpy()
    stats = aux["stats"].cpu().numpy()
    cnt = counts.cpu().numpy()
    n_act, n_inact, alg_bytes, per_act, per_inact = _alg_bytes(cfg, adv, lens)
    for _ in range(warmup):
        dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, **kw)
    torch.cuda.synchronize()
    # per-row-kernel events on the stream the library launches on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:  # create the underlying HIP events
        e0.record()
        e1.record()
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(steps):
        cev[k].record()
        dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, rows_events=evs[k], **kw)
    cev[steps].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = cev[0].elapsed_time(cev[steps])
    call_ms = [cev[k].elapsed_time(cev[k + 1]) for k in range(steps)]
    rows_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    rows_avg = float(np.mean(rows_ms))
    if dr.device_status(ws) != dr.OK:
        raise SystemExit("device status not OK")
    achieved = alg_bytes / (rows_avg / 1e3) / 1e9
    out = {
        "workload": cfg.name, "B": cfg.B, "G": cfg.G, "C": cfg.C, "V": cfg.V, "dtype": cfg.dtype,
        "token_rows": cfg.T, "beta": cfg.beta, "eps": cfg.eps, "norm_const": cfg.norm_const,
        "active_rows": n_act, "inactive_rows": n_inact, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_total / steps, "tokens_per_s": cfg.T / (ms_total / steps / 1e3),
        "valid_tokens_per_s": float(cnt[0]) / (ms_total / steps / 1e3),
        "call_ms": _spread(call_ms), "k_rows_ms": _spread(rows_ms), "k_rows_ms_mean": rows_avg,
        "alg_bytes_per_launch": alg_bytes, "bytes_per_active_row": per_act,
        "bytes_per_inactive_row": per_inact, "achieved_gbps": achieved,
        "frac": achieved / HBM_PEAK_GBPS, "traffic": _traffic(cfg.name),
        "wall_s_timed": wall,
        "rollout_stats": {
            "groups": cfg.B, "groups_without_contrast": int(stats[0]),
            "contrast_frac": 1.0 - float(stats[0]) / cfg.B,
            "useful_groups_per_s": (cfg.B - float(stats[0])) / (ms_total / steps / 1e3),
            "rows_without_eos": int(stats[1]), "truncation_rate": float(stats[1]) / cfg.N,
            "mean_completion_len": float(cnt[0]) / cfg.N, "counted_tokens": int(cnt[0]),
            "active_tokens": int(cnt[1]), "ratio_outside_clip": int(stats[2]),
            "clip_cut_tokens": int(stats[3])},
    }
    if ceilings and cfg.dtype == "bf16":
        rb = cfg.V * 2
        mask = np.arange(cfg.C)[None, :] < lens[:, None]
        active = (mask & ((adv[:, None] != 0) | (cfg.beta != 0))).reshape(-1).astype(np.uint8)
        act_t = torch.from_numpy(active).to(dev)
        sink = torch.zeros(cfg.T, dtype=torch.int32, device=dev)
        stride = _row_stride(cfg.T)
        full = 2 * cfg.T * rb
        t_copy = _timed_ceiling(0, logits, dlogits, cfg.T, rb, 1, None, sink)
        t_fill = _timed_ceiling(1, None, dlogits, cfg.T, rb, 1, None, sink)
        t_read = _timed_ceiling(2, logits, dlogits, cfg.T, rb, 1, None, sink)
        t_stride = _timed_ceiling(0, logits, dlogits, cfg.T, rb, stride, act_t, sink)
        order = np.concatenate([np.flatnonzero(active), np.flatnonzero(active == 0)])
        class_rows = torch.from_numpy(order.astype(np.int32)).to(dev)
        counters = torch.zeros(65, dtype=torch.int32, device=dev)
        t_skel = _timed_ceiling(0, logits, dlogits, cfg.T, rb, stride, act_t, sink,
                                ticket=(class_rows, int(active.sum()), counters))
        skel_bytes = n_act * 2 * rb + n_inact * rb
        out["ceilings"] = {
            "how": "libceiling.so: one 1024-thread workgroup per row, every 16-byte load of a "
                   "row in flight, nontemporal loads, sc1|nt buffer stores (the row kernel's "
                   "access pattern, no arithmetic), on the same logits / dlogits buffers; "
                   "median of 5 launches timed by dispatch events",
            "copy_gbps": full / (t_copy / 1e3) / 1e9,
            "fill_gbps": cfg.T * rb / (t_fill / 1e3) / 1e9,
            "read_gbps": cfg.T * rb / (t_read / 1e3) / 1e9,
            "skeleton": {"what": "this batch's active rows copied and zero rows filled, in the "
                                 "row kernel's ticket order: its data movement alone",
                         "ms": t_skel, "gbps": skel_bytes / (t_skel / 1e3) / 1e9,
                         "k_rows_frac_of_skeleton": t_skel / rows_avg},
            "skeleton_stride_order": {
                "what": "the same movement with workgroup b owning row (b * stride) mod T "
                        "(the row kernel's earlier order)",
                "ms": t_stride, "gbps": skel_bytes / (t_stride / 1e3) / 1e9},
            "k_rows_frac_of_copy": achieved / (full / (t_copy / 1e3) / 1e9),
        }
    # the forward-only log-prob pass (old / reference log-probs) over the same
    # logits: every row read once, one binary32 per row written
    lp_ms = _timed_calls(lambda: dr.logprobs(logits, tokens))
    lp_bytes = cfg.T * (cfg.V * logits.element_size() + 8 + 4)
    out["logprobs_pass"] = {
        "entry_point": "drgrpo_logprobs", "ms": lp_ms, "bytes_per_call": lp_bytes,
        "gbps": lp_bytes / (lp_ms["median"] / 1e3) / 1e9,
        "frac": lp_bytes / (lp_ms["median"] / 1e3) / 1e9 / HBM_PEAK_GBPS}
    if eager:
        loss_t, _ = dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, **kw)
        e = eager_loss(cfg, logits, tokens, rewards, old, ref, float(loss_t.item()), dlogits)
        e["speedup_of_fused_call"] = e["ms"] / float(np.median(call_ms))
        out["torch_eager"] = e
    del kw, aux, logits, dlogits, ws, old, ref
    torch.cuda.empty_cache()
    return out


def run_decode(name, args):
    """Decode attention of the rollout step: one new token per sequence against
    its bfloat16 KV cache (S sequences, grouped-query heads).  A decode loop
    runs the call once per layer, each on that layer's cache, so the timed
    graph cycles through distinct caches (at least 1 GB of them, four times
    the on-die caches) and every call reads its keys and values from HBM; the
    same calls on one cache (warm) are reported beside it."""
    import math

    import numpy as np
    import torch

    from synth.attention import get_decode_config, make_decode_case
    import synth
    from synth import attention as sa
    import rl_post_loss_dr_amd as dr

    c = get_decode_config(name)
    dev = torch.device("cuda:0")
    per_layer = 2 * c.S * c.Hkv * c.Lmax * c.D * 2
    NL = max(2, min(64, math.ceil(1e9 / per_layer)))
    q = torch.empty((c.S, c.Hq, c.D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((NL, c.S, c.Hkv, c.Lmax, c.D), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    synth.gpu_normal_fill(q, c.seed, sa.S_QUERY, 0, c.std)
    synth.gpu_normal_fill(k, c.seed, sa.S_KEY, 0, c.std)
    synth.gpu_normal_fill(v, c.seed, sa.S_VALUE, 0, c.std)
    lens_h = make_decode_case(c).lens if c.ragged else np.full(c.S, c.Lmax, np.int32)
    lens = torch.from_numpy(lens_h).to(dev)
    ws = torch.empty(dr.decode_attention_workspace_bytes(c.S, c.Hq, c.Hkv, c.Lmax, c.D),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((c.S, c.Hq, c.D), dtype=torch.bfloat16, device=dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def calls(cold):
        for layer in range(NL):
            j = layer if cold else 0
            dr.decode_attention(q, k[j], v[j], lens, workspace=ws, out=out)

    for _ in range(max(1, args.warmup // NL)):
        calls(True)
    torch.cuda.synchronize()
    reps = max(1, args.steps // NL)
    t0.record()
    for _ in range(reps):
        calls(True)
    t1.record()
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1) / (reps * NL)
    # A decode loop replays its step from a captured graph; launched one by one
    # from Python a call costs ~9 us of host time, more than the kernel.
    res = {}
    for cold in (True, False):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            calls(cold)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            calls(cold)
        graph.replay()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            graph.replay()
        t1.record()
        torch.cuda.synchronize()
        res[cold] = t0.elapsed_time(t1) / (reps * NL)
    ms, ms_warm = res[True], res[False]
    # algorithmic bytes: the cached keys and values read once, queries, outputs, lengths
    kv = 2 * c.Hkv * c.D * 2 * int(lens_h.clip(0, c.Lmax).sum())
    alg = kv + 2 * 2 * c.S * c.Hq * c.D + 4 * c.S
    gbps = alg / (ms / 1e3) / 1e9
    return {
        "metric": "decode attention tokens/s and HBM GB/s (% of peak)", "value": c.S / (ms / 1e3),
        "unit": "decoded tokens/s", "n_gpus": 1, "steps": reps * NL, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded generator; no weights)",
        "config": {"workload": c.name, "S": c.S, "Hq": c.Hq, "Hkv": c.Hkv, "D": c.D,
                   "Lmax": c.Lmax, "caches_cycled": NL},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "whole call (k_attn_fused, + k_attn_combine when split), "
                               "replayed from a captured graph over distinct caches",
                     "alg_bytes_per_call": alg},
        "ms_per_step_warm": ms_warm,
        "ms_per_step_eager": ms_eager,
        "note": "ms_per_step: calls on caches_cycled distinct caches replayed from a captured "
                "graph, each reading its cache from HBM (device time per call); "
                "ms_per_step_warm: the same calls all on one cache (kept in the on-die caches); "
                "ms_per_step_eager: the cold calls launched one by one from Python",
        "device": torch.cuda.get_device_name(0),
    }


def run_rollout(name, args):
    """The rollout step with the decode attention integrated: one decode step
    of a Qwen2.5-0.5B-shaped policy (24 layers, random weights) for S
    sequences at L cached positions, eager and replayed from a captured graph,
    beside the attention call alone on a layer's cache of the same shape."""
    import torch

    import rl_post_loss_dr_amd as dr
    from rl_post_loss_dr_amd.rollout import QWEN25_05B, DecodePolicy

    sizes = {"rollout_s64_l512": (64, 512)}
    if name not in sizes:
        raise SystemExit(f"unknown rollout workload {name}: {sorted(sizes)}")
    S, L = sizes[name]
    sh = QWEN25_05B
    dev = torch.device("cuda:0")
    pol = DecodePolicy(sh, S, L + 64, seed=7401, device=dev)
    pol.fill_cache(7402)
    g = torch.Generator(device=dev)
    g.manual_seed(7403)
    tok = torch.randint(0, sh.vocab, (S,), device=dev, generator=g)
    # every step writes position L-1 and attends over L positions (the same
    # work each time; a rollout advances the position, which the graph test
    # covers)
    pos = torch.full((S,), L - 1, dtype=torch.int32, device=dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        pol.step(tok, pos)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        pol.step(tok, pos)
    ev1.record()
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / args.steps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pol.step(tok, pos)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pol.step(tok, pos)
    graph.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same step with the rotary embedding and the cache append in PyTorch
    # around the plain attention call (graph-replayed as well)
    with torch.cuda.stream(side):
        pol.step(tok, pos, attention="library_unfused")
    torch.cuda.current_stream().wait_stream(side)
    graph_u = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_u):
        pol.step(tok, pos, attention="library_unfused")
    graph_u.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        graph_u.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_unfused = ev0.elapsed_time(ev1) / args.steps
    # the attention call alone on layer 0's cache (graph of 20 calls replayed)
    q = torch.randn((S, sh.heads, sh.head_dim), generator=g, device=dev).to(torch.bfloat16)
    lens = pos + 1
    ws = torch.empty(dr.decode_attention_workspace_bytes(S, sh.heads, sh.kv_heads, L + 64,
                                                         sh.head_dim),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    args_a = (q, pol.k_cache[0], pol.v_cache[0], lens)
    dr.decode_attention(*args_a, workspace=ws, out=out)
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for _ in range(20):
            dr.decode_attention(*args_a, workspace=ws, out=out)
    ga.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(5):
        ga.replay()
    ev1.record()
    torch.cuda.synchronize()
    attn_ms = ev0.elapsed_time(ev1) / 100
    # algorithmic bytes per step: every weight once (the output projection is
    # the tied embedding), the cached keys and values once, the new keys and
    # values and the logits written
    n_w = pol.embed.numel() + sum(t.numel() for L_ in pol.layers for t in L_.values()) + \
        pol.ln_f.numel()
    kv_read = sh.layers * 2 * S * sh.kv_heads * L * sh.head_dim * 2
    alg = 2 * n_w + kv_read + sh.layers * 2 * S * sh.kv_heads * sh.head_dim * 2 + S * sh.vocab * 2
    gbps = alg / (ms / 1e3) / 1e9
    return {
        "metric": "rollout decode step tokens/s (decode attention integrated)",
        "value": S / (ms / 1e3), "unit": "decoded tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights of the Qwen2.5-0.5B shape; random cache)",
        "config": {"workload": name, "S": S, "cached_positions": L, "layers": sh.layers,
                   "hidden": sh.hidden, "heads": sh.heads, "kv_heads": sh.kv_heads,
                   "head_dim": sh.head_dim, "vocab": sh.vocab},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "whole decode step (all layers), replayed from a captured graph",
                     "alg_bytes_per_step": alg, "weight_bytes": 2 * n_w,
                     "kv_cache_bytes_read": kv_read},
        "ms_per_step_eager": ms_eager,
        "ms_per_step_unfused_rope_append": ms_unfused,
        "attention_standalone_ms_per_layer": attn_ms,
        "attention_standalone_share": sh.layers * attn_ms / ms,
        "note": "ms_per_step: the step replayed from a captured graph, its attention block "
                "(rotary embedding, cache append, attention) one library call; "
                "ms_per_step_eager: launched op by op from Python; "
                "ms_per_step_unfused_rope_append: graph-replayed with the rotary embedding and "
                "the append in PyTorch around the attention call; attention_standalone: the "
                "attention call on one layer's cache replayed alone (the in-loop kernel times "
                "are in the rocprofv3 summary)",
        "device": torch.cuda.get_device_name(0),
    }


def synth_perturb(lp, noise):
    import synth

    return synth.perturb(lp, noise)


EXTRA_LOSS = ["qwen_b8g16c512", "qwen_kl_b16g8c1024", "qwen_dense_b8g8c256"]
EXTRA_STEPS = {"qwen_b8g16c512": 10, "qwen_kl_b16g8c1024": 10, "qwen_dense_b8g8c256": 20}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_b8g8c256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads, the ceilings and the eager PyTorch timing")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip timing the plain eager PyTorch formulation (context only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 4 GiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if args.calibrate_copy:
        # a plain copy kernel of known size: 4 GiB read + 4 GiB written per call
        n = 1 << 31
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 2 * n, "calibrate_copy_bytes_written": 2 * n,
                          "calls": 3}), flush=True)
        return

    if args.workload.startswith("decode_"):
        print(json.dumps(run_decode(args.workload, args)), flush=True)
        return
    if args.workload.startswith("rollout_"):
        print(json.dumps(run_rollout(args.workload, args)), flush=True)
        return
    cfg = synth.get_config(args.workload)
    case = synth.make_case(cfg)
    if cfg.H is not None:
        r = measure_lmhead(cfg, case, args.steps, args.warmup, eager=not args.no_eager)
        rec = {
            "metric": METRIC, "value": r["tokens_per_s"], "unit": "completion tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded generator; no dataset or weights)",
            "config": {k: r[k] for k in ("workload", "B", "G", "C", "V", "H", "token_rows",
                                         "active_tokens")},
            "roofline": {"bound": "mfma", "achieved": r["forward_product"]["tflops"],
                         "peak": 2500.0, "unit": "TFLOP/s", "frac": r["forward_product"]["frac"],
                         "traffic": None, "kernel": "k_gemm<GM_LSE> (forward log-sum-exp product)",
                         "kernel_ms": r["forward_product"]["ms"]["median"]},
            "lmhead": r, "provenance": provenance(cfg.seed),
        }
        print(json.dumps(rec), flush=True)
        return

    head = measure_loss(cfg, case, args.steps, args.warmup, ceilings=not args.headline_only,
                        eager=not (args.headline_only or args.no_eager))
    rec = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "completion tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "G": cfg.G, "C": cfg.C, "V": cfg.V,
                   "token_rows": cfg.T, "beta": cfg.beta, "eps": cfg.eps,
                   "norm_const": cfg.norm_const, "active_rows": head["active_rows"],
                   "inactive_rows": head["inactive_rows"]},
        "roofline": {"bound": "hbm", "achieved": head["achieved_gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": head["frac"], "traffic": head["traffic"],
                     "kernel": "k_rows", "kernel_ms": head["k_rows_ms_mean"],
                     "alg_bytes_per_launch": head["alg_bytes_per_launch"],
                     "bytes_per_active_row": head["bytes_per_active_row"],
                     "bytes_per_inactive_row": head["bytes_per_inactive_row"]},
        "step_gbps_alg": head["alg_bytes_per_launch"] / (head["ms_per_step"] / 1e3) / 1e9,
        "call_ms": head["call_ms"],
        "k_rows_ms": head["k_rows_ms"],
        "valid_tokens_per_s": head["valid_tokens_per_s"],
        "rollout_stats": head["rollout_stats"],
        "wall_s_timed": head["wall_s_timed"],
    }
    if "ceilings" in head:
        rec["ceilings"] = head["ceilings"]
    rec["logprobs_pass"] = head["logprobs_pass"]
    if "torch_eager" in head:
        rec["torch_eager"] = head["torch_eager"]
    rec["provenance"] = provenance(cfg.seed)
    if not args.headline_only and cfg.name == "qwen_b8g8c256":
        work = {}
        for name in EXTRA_LOSS:
            c = synth.get_config(name)
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            r = measure_loss(c, synth.make_case(c), EXTRA_STEPS[name], 3,
                             ceilings=name == "qwen_dense_b8g8c256")
            r.pop("rollout_stats", None)
            work[name] = r
        c = synth.get_config("lmhead_b8g8c512")
        print(f"[bench] {c.name}", file=sys.stderr, flush=True)
        work[c.name] = measure_lmhead(c, synth.make_case(c), 5, 2, eager=not args.no_eager)
        rec["workloads"] = work
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, case)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
