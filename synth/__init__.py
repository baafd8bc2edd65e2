"""Seeded synthetic inputs for the Dr. GRPO loss (shared by the oracle side and
the GPU side; holds none of the loss arithmetic).

Every random value is a pure function of (seed, stream, index) through the
counter-based generator defined in ``synth_rng.h`` (SplitMix64 mixing of a
Weyl sequence).  Three bit-identical implementations exist:

* ``libsynth_cpu.so`` (gcc, OpenMP) fills host buffers with normal values;
* ``libsynth_gpu.so`` (hipcc, gfx950) fills device buffers with the same values;
* the numpy functions below generate the small per-row / per-token arrays
  (token ids, EOS placement, rewards, log-prob noise) and mirror the C code
  for cross-checking.

Normal values use the Irwin-Hall(12) approximation of N(0, s^2) (mean 0,
std s, support +-6 s), chosen because it is exact integer arithmetic followed
by one rounded multiply, so CPU and GPU agree bit for bit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .configs import CONFIGS, Config, get_config  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

# Stream numbers: one independent stream per kind of synthetic value.
S_LOGITS, S_TOKENS, S_EOS_ROWS, S_EOS_POS, S_REWARDS = 1, 2, 3, 4, 5
S_OLD_NOISE, S_REF_NOISE, S_HIDDEN, S_WEIGHT = 6, 7, 8, 9

F32, BF16 = 0, 1

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_SALT = 0x632BE59BD9B4E019


# --------------------------------------------------------------------------- build
def build(verbose: bool = False) -> None:
    """Compile the host generator with gcc and the device generator with hipcc."""
    cpu = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-o", CPU_LIB, os.path.join(_HERE, "synth_cpu.c")]
    gpu = ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", GPU_LIB, os.path.join(_HERE, "synth_gpu.hip")]
    for cmd in (cpu, gpu):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)


_cpu = None
_gpu = None


def _cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            raise RuntimeError(f"{CPU_LIB} is not built; run synth.build()")
        lib = ctypes.CDLL(CPU_LIB)
        lib.synth_cpu_fill_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                              ctypes.c_void_p]
        lib.synth_cpu_fill_normal.restype = ctypes.c_int
        lib.synth_cpu_fill_normal_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.synth_cpu_fill_normal_rows.restype = ctypes.c_int
        _cpu = lib
    return _cpu


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run synth.build()")
        lib = ctypes.CDLL(GPU_LIB)
        lib.synth_gpu_fill_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_gpu_fill_normal.restype = ctypes.c_int
        _gpu = lib
    return _gpu


# ------------------------------------------------------------ numpy mirror of synth_rng.h
def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def key(seed: int, stream: int) -> np.uint64:
    s = int(mix64(np.array([seed & _M64], dtype=np.uint64))[0])
    t = (stream * _GAMMA + _SALT) & _M64
    return mix64(np.array([s ^ t], dtype=np.uint64))[0]


def draws(k: np.uint64, counters) -> np.ndarray:
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(k) + (c + np.uint64(1)) * np.uint64(_GAMMA))


def ih12_num(k: np.uint64, idx) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    s = np.zeros(idx.shape, dtype=np.int64)
    for j in range(3):
        with np.errstate(over="ignore"):
            d = draws(k, np.uint64(3) * idx + np.uint64(j))
        for sh in (0, 16, 32, 48):
            s += ((d >> np.uint64(sh)) & np.uint64(0xFFFF)).astype(np.int64)
    return s - 393210


def normal64(seed: int, stream: int, idx, stdev: float) -> np.ndarray:
    """N(0, stdev^2) values as float64 (exact numerator / 65536, times stdev)."""
    return (ih12_num(key(seed, stream), idx).astype(np.float64) * (1.0 / 65536.0)) * stdev


def normal32(seed: int, stream: int, idx, stdev: float) -> np.ndarray:
    """The binary32 values synth_normal_f32 produces."""
    return normal64(seed, stream, idx, stdev).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform01(seed: int, stream: int, counters) -> np.ndarray:
    """53-bit uniforms in [0, 1)."""
    d = draws(key(seed, stream), counters)
    return (d >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def randint(seed: int, stream: int, counters, n: int) -> np.ndarray:
    """Integers in [0, n) (draw modulo n; bias below 2^-40 for n < 2^24)."""
    return (draws(key(seed, stream), counters) % np.uint64(n)).astype(np.int64)


# ---------------------------------------------------------------------- bulk normals
def cpu_normal(seed: int, stream: int, offset: int, n: int, stdev: float, dtype: int) -> np.ndarray:
    """Host array of n generated values starting at global element `offset`."""
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    rc = _cpu_lib().synth_cpu_fill_normal(seed, stream, offset, n, stdev, dtype,
                                         out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"synth_cpu_fill_normal failed ({rc})")
    return out


def cpu_normal_rows(seed: int, stream: int, rows, row_len: int, stdev: float,
                    dtype: int) -> np.ndarray:
    """Rows `rows` of a generated [*, row_len] tensor, as a [len(rows), row_len] host array."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, row_len), dtype=np.float32 if dtype == F32 else np.uint16)
    rc = _cpu_lib().synth_cpu_fill_normal_rows(seed, stream, rows.ctypes.data, rows.size,
                                              row_len, stdev, dtype, out.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"synth_cpu_fill_normal_rows failed ({rc})")
    return out


def gpu_normal_fill(tensor, seed: int, stream: int, offset: int, stdev: float) -> None:
    """Fill a contiguous CUDA tensor (float32 or bfloat16) in place on its current stream."""
    import torch

    if not tensor.is_cuda or not tensor.is_contiguous():
        raise ValueError("gpu_normal_fill needs a contiguous device tensor")
    if tensor.dtype == torch.float32:
        dt = F32
    elif tensor.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise ValueError(f"unsupported dtype {tensor.dtype}")
    s = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _gpu_lib().synth_gpu_fill_normal(seed, stream, offset, tensor.numel(), stdev, dt,
                                         tensor.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_normal failed ({rc})")


from .inputs import Case, make_case, perturb  # noqa: E402,F401
