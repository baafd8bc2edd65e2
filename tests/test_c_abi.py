"""The C ABI from a C caller: tests/c_abi/abi_from_c.c includes
include/drgrpo.h as C11 under -pedantic -Werror and links against
libdrgrpo.so.  On the CPU its sizes and rejections equal the Python
binding's; on the GPU a call driven by nothing but the HIP runtime API gives
the binding's loss and dlogits bit for bit (the same library underneath)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import rl_post_loss_dr_amd as dr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c")
PKG = os.path.dirname(dr.LIB)


def _build(tmp):
    if not os.path.exists(dr.LIB):
        pytest.skip("libdrgrpo.so is not built")
    out = os.path.join(str(tmp), "abi_from_c.so")
    cmd = ["gcc", "-std=c11", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-isystem", "/opt/rocm/include", "-o", out, SRC, "-L", PKG, "-ldrgrpo",
           "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return ctypes.CDLL(out)


def test_header_compiles_as_c_and_host_checks_agree(tmp_path):
    c = _build(tmp_path)
    c.c_abi_host_checks.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_void_p, ctypes.c_char_p,
                                                          ctypes.c_size_t]
    out = np.zeros(7, np.int64)
    text = ctypes.create_string_buffer(128)
    N, C, V, G = 64, 256, 151936, 8
    assert c.c_abi_host_checks(N, C, V, G, out.ctypes.data, text, 128) == 0
    assert out[0] == dr.workspace_bytes(N, C, V, G) > 0
    assert out[1] == 0
    assert list(out[2:]) == [dr.ERR_NULL, dr.ERR_DTYPE, dr.ERR_SHAPE, dr.ERR_PARAM,
                             dr.ERR_WORKSPACE]
    assert text.value == dr.lib().drgrpo_status_string(dr.ERR_DTYPE)


@pytest.mark.gpu
def test_loss_from_c_matches_the_binding(tmp_path):
    import torch

    from _cases import small_case, compare_loss

    c = _build(tmp_path)
    P = ctypes.c_void_p
    c.c_abi_loss.argtypes = [P, P, ctypes.c_int64, P, P, ctypes.c_int64, ctypes.c_int64,
                             ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float, P, P]
    cfg, case, x, old, ref, res = small_case("mini_bf16")
    assert cfg.dtype == "bf16" and ref is None and cfg.beta == 0.0
    x = np.ascontiguousarray(x.reshape(cfg.N, cfg.C, cfg.V)).view(np.uint16)
    tok = np.ascontiguousarray(case.tokens, dtype=np.int64)
    rew = np.ascontiguousarray(case.rewards, dtype=np.float32)
    old = np.ascontiguousarray(old, dtype=np.float32)
    loss_c = np.zeros(1, np.float32)
    dl_c = np.zeros_like(x)
    rc = c.c_abi_loss(x.ctypes.data, tok.ctypes.data, cfg.eos_id, rew.ctypes.data, old.ctypes.data,
                      cfg.N, cfg.C, cfg.V, cfg.G, cfg.eps, cfg.norm_const, loss_c.ctypes.data,
                      dl_c.ctypes.data)
    assert rc == 0, rc
    dev = torch.device("cuda:0")
    logits = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    loss_p, dl_p = dr.loss_fwd_bwd(logits, torch.from_numpy(tok).to(dev), cfg.eos_id,
                                   torch.from_numpy(rew).to(dev), torch.from_numpy(old).to(dev),
                                   None, G=cfg.G, eps=cfg.eps, norm_const=cfg.norm_const)
    torch.cuda.synchronize()
    assert loss_c[0].view(np.uint32) == np.float32(loss_p.item()).view(np.uint32)
    assert np.array_equal(dl_c.view(np.uint16),
                          dl_p.view(torch.int16).cpu().numpy().view(np.uint16))
    compare_loss(cfg, float(loss_c[0]), res)
