"""Benchmark of the fused Dr. GRPO loss forward + backward on one MI355X.

One step = one drgrpo_loss_fwd_bwd call (completion mask, group advantage,
log-prob sweep over the vocabulary, clipped surrogate, token sum, dlogits)
over one synthetic rollout batch resident in HBM.  Prints ONE JSON line.

Default workload: B=8 prompts x G=8 completions x C=256 tokens over the
151,936-entry vocabulary in bfloat16 (the Qwen2.5-0.5B-Instruct-shaped
batch), synthetic seeded inputs.  logp_old is the library's own forward
log-prob plus N(0, 0.02^2) noise, as an update step would receive it.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
    h = hashlib.sha256()
    for p in ("rl_post_loss_dr_amd/csrc/drgrpo.hip", "rl_post_loss_dr_amd/csrc/common.h"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(workload):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/), if the
    committed measurement was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"k_rows_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("src_hash") != _src_hash():
        return None
    return rec.get("bytes_per_launch")


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
    host = {"nproc": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            host["cpu_model"] = next(l.split(":", 1)[1].strip() for l in f
                                     if l.startswith("model name"))
        with open("/proc/meminfo") as f:
            host["ram_gb"] = round(int(next(l for l in f if l.startswith("MemTotal")).split()[1])
                                   / 2 ** 20, 1)
    except (OSError, StopIteration):
        pass
    return {"value": tok_s, "unit": "completion tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} token rows (every {step}th of {T}) x V={cfg.V}, "
                      f"{reps} passes in {el:.1f} s; mask and advantage over the whole batch",
            "single_thread": single, "host": host}


def run_lmhead(cfg, case, args):
    """Fused lm_head workload: hidden [T, H] and W [V, H] in, loss, dhidden, dW out."""
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
    for _ in range(args.warmup):
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, old, None, **kw)
    torch.cuda.synchronize()
    # forward-product events on the stream the library launches on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for k in range(args.steps):
        dr.lmhead_loss_fwd_bwd(hidden, W, tokens, cfg.eos_id, rewards, old, None,
                               fwd_events=evs[k], **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    per_gemm = 2.0 * n_act * cfg.V * cfg.H  # one product over the active tokens
    achieved = per_gemm / (fwd_ms / 1e3) / 1e12
    return {
        "metric": METRIC, "value": cfg.T / (ms / 1e3), "unit": "completion tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "G": cfg.G, "C": cfg.C, "V": cfg.V,
                   "H": cfg.H, "token_rows": cfg.T, "active_tokens": n_act},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": achieved / 2500.0, "traffic": None,
                     "kernel": "k_gemm<GM_LSE> (forward log-sum-exp product)",
                     "kernel_ms": fwd_ms, "alg_flops_per_launch": per_gemm},
        "call_tflops_required": 3 * per_gemm / (ms / 1e3) / 1e12,
        "call_tflops_executed": 4 * per_gemm / (ms / 1e3) / 1e12,
        "note": "required = logits, dhidden, dW products over the active tokens; executed "
                "adds the logits recompute of the backward chunks",
        "device": torch.cuda.get_device_name(0),
    }


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_b8g8c256")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 4 GiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import rl_post_loss_dr_amd as dr

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
        print(json.dumps(run_lmhead(cfg, case, args)), flush=True)
        return
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
    dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, aux=aux, **kw)
    torch.cuda.synchronize()
    lens = aux["len"].cpu().numpy()
    adv = aux["adv"].cpu().numpy()
    stats = aux["stats"].cpu().numpy()
    n_act, n_inact, alg_bytes, per_act, per_inact = _alg_bytes(cfg, adv, lens)

    for _ in range(args.warmup):
        dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, **kw)
    torch.cuda.synchronize()

    # per-row-kernel events on the stream the library launches on
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:  # create the underlying HIP events
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    # whole-call events between the calls (median / min per call)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for k in range(args.steps):
        cev[k].record()
        dr.loss_fwd_bwd(logits, tokens, cfg.eos_id, rewards, old, ref, rows_events=evs[k], **kw)
    cev[args.steps].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    call_ms = [cev[k].elapsed_time(cev[k + 1]) for k in range(args.steps)]
    rows_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    rows_ms_avg = float(np.mean(rows_ms))
    if dr.device_status(ws) != dr.OK:
        raise SystemExit("device status not OK")
    # a plain device copy of the logits into the dlogits buffer on the same
    # box (read + write of N*C*V elements), after the timed region
    copy_bytes = 2 * logits.numel() * logits.element_size()
    for _ in range(2):
        dlogits.copy_(logits)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dlogits.copy_(logits)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = copy_bytes / (c0.elapsed_time(c1) / 5 / 1e3) / 1e9

    tok_s = cfg.T / (ms_step / 1e3)
    achieved = alg_bytes / (rows_ms_avg / 1e3) / 1e9
    traffic = _traffic(args.workload)
    rec = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "completion tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {"workload": cfg.name, "B": cfg.B, "G": cfg.G, "C": cfg.C, "V": cfg.V,
                   "token_rows": cfg.T, "beta": cfg.beta, "eps": cfg.eps,
                   "norm_const": cfg.norm_const, "active_rows": n_act, "inactive_rows": n_inact},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "k_rows", "kernel_ms": rows_ms_avg,
                     "alg_bytes_per_launch": alg_bytes, "bytes_per_active_row": per_act,
                     "bytes_per_inactive_row": per_inact},
        "step_gbps_alg": alg_bytes / (ms_step / 1e3) / 1e9,
        "call_ms_median": float(np.median(call_ms)),
        "call_ms_min": float(np.min(call_ms)),
        "k_rows_ms_median": float(np.median(rows_ms)),
        "k_rows_ms_min": float(np.min(rows_ms)),
        "valid_tokens_per_s": float(stats[4]) / (ms_step / 1e3),
        "copy_ref": {"gbps": copy_gbps, "bytes_per_call": copy_bytes,
                     "how": "torch copy_ of the logits tensor into the dlogits tensor",
                     "k_rows_frac_of_copy": achieved / copy_gbps},
        "rollout_stats": {
            "groups": cfg.B, "groups_without_contrast": int(stats[0]),
            "contrast_frac": 1.0 - float(stats[0]) / cfg.B,
            "useful_groups_per_s": (cfg.B - float(stats[0])) / (ms_step / 1e3),
            "rows_without_eos": int(stats[1]), "truncation_rate": float(stats[1]) / cfg.N,
            "mean_completion_len": float(stats[4]) / cfg.N, "counted_tokens": int(stats[4]),
            "active_tokens": int(stats[5]), "ratio_outside_clip": int(stats[2]),
            "clip_cut_tokens": int(stats[3])},
        "wall_s_timed": wall,
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, case)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
