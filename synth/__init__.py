"""Seeded synthetic inputs for the W6A6 / W6A8 linear-layer workloads.

This module draws the fp16 weight and activation tensors that both the CPU
oracle and the GPU library consume.  It contains no step of the quantization
method itself.  Distributions follow the LLaMA-shaped linear-layer workloads:

* weights  W[N][K] ~ N(0, 0.02), rounded to fp16;
* activations X[M][K] ~ N(0, 1), with round(0.01*K) input channels (column
  indices k, the same for every token) multiplied by 20 before fp16 rounding,
  which models the outlier channels of LLM activations.

The bit generator is counter based (splitmix64 output c for state `seed`),
implemented in ``synth.c``; every tensor gets its own seed derived from a base
seed and a label tuple with :func:`derive_seed`.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

BASE_SEED = 20250806
W_SIGMA = 0.02
X_SIGMA = 1.0
OUTLIER_FRACTION = 0.01
OUTLIER_SCALE = 20.0


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    import subprocess

    src = os.path.join(_HERE, "synth.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", src, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.synth_rand64.restype = ctypes.c_uint64
    lib.synth_rand64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.synth_f64_to_f16.restype = ctypes.c_uint16
    lib.synth_f64_to_f16.argtypes = [ctypes.c_double]
    lib.synth_normal_f16.restype = None
    lib.synth_normal_f16.argtypes = [
        ctypes.c_uint64, ctypes.c_double, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
    _lib = lib
    return lib


def _mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def rand64(seed: int, c: int) -> int:
    """splitmix64 output number ``c`` for initial state ``seed`` (pure Python)."""
    return _mix64((seed + (c + 1) * GOLDEN) & MASK64)


def derive_seed(*labels) -> int:
    """Fold a tuple of ints / strings into one 64-bit seed."""
    h = 0x243F6A8885A308D3
    for lab in labels:
        if isinstance(lab, str):
            v = 0
            for ch in lab.encode():
                v = _mix64(v ^ ch ^ (v << 8))
        else:
            v = int(lab) & MASK64
        h = _mix64(h ^ _mix64(v + GOLDEN))
    return h


def default_threads() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return max(1, min(n, 16))


def outlier_channels(seed: int, K: int, fraction: float = OUTLIER_FRACTION) -> np.ndarray:
    """round(fraction*K) distinct column indices by a seeded partial Fisher-Yates shuffle."""
    count = int(round(fraction * K))
    perm = np.arange(K, dtype=np.int64)
    for i in range(count):
        j = i + rand64(seed, i) % (K - i)
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def normal_f16(seed: int, rows: int, cols: int, sigma: float,
               outlier_cols: np.ndarray | None = None,
               outlier_scale: float = OUTLIER_SCALE, nthreads: int | None = None,
               out: np.ndarray | None = None) -> np.ndarray:
    """[rows][cols] fp16 (returned as a numpy float16 array)."""
    lib = _load()
    if out is None:
        out = np.empty((rows, cols), dtype=np.float16)
    assert out.dtype == np.float16 and out.flags.c_contiguous and out.size == rows * cols
    flags_ptr = None
    if outlier_cols is not None and len(outlier_cols):
        flags = np.zeros(cols, dtype=np.uint8)
        flags[np.asarray(outlier_cols, dtype=np.int64)] = 1
        flags_ptr = flags.ctypes.data
    else:
        flags = None
    lib.synth_normal_f16(seed & MASK64, float(sigma), rows, cols, flags_ptr,
                         float(outlier_scale), out.ctypes.data,
                         nthreads if nthreads is not None else default_threads())
    return out


def weights(seed: int, N: int, K: int, sigma: float = W_SIGMA, **kw) -> np.ndarray:
    """W[N][K] ~ N(0, sigma) in fp16."""
    return normal_f16(seed, N, K, sigma, **kw)


def activations(seed: int, M: int, K: int, sigma: float = X_SIGMA,
                fraction: float = OUTLIER_FRACTION, scale: float = OUTLIER_SCALE,
                **kw) -> np.ndarray:
    """X[M][K] ~ N(0, sigma) with round(fraction*K) outlier columns scaled by `scale`."""
    cols = outlier_channels(derive_seed(seed, "outliers"), K, fraction)
    return normal_f16(seed, M, K, sigma, outlier_cols=cols, outlier_scale=scale, **kw)


# ---------------------------------------------------------------------------
# Workload tables: LLaMA-2 linear-layer shapes (hidden, intermediate, GQA kv).
# ---------------------------------------------------------------------------

GROUP = 128

LLAMA2_7B = {"qkv": (12288, 4096), "o": (4096, 4096),
             "gate_up": (22016, 4096), "down": (4096, 11008)}
LLAMA2_13B = {"qkv": (15360, 5120), "o": (5120, 5120),
              "gate_up": (27648, 5120), "down": (5120, 13824)}
LLAMA2_70B = {"qkv": (10240, 8192), "o": (8192, 8192),
              "gate_up": (57344, 8192), "down": (8192, 28672)}

WORKLOADS = {
    "toy_w6a6": {"layers": {"toy": (256, 512)}, "M": (16,), "abits": (6,)},
    "llama2_7b_w6a6": {"layers": LLAMA2_7B, "M": (1, 16, 128), "abits": (6,)},
    "llama2_13b_w6a8": {"layers": LLAMA2_13B, "M": (1, 64, 512), "abits": (8,)},
    "llama2_70b_w6a6_w6a8": {"layers": LLAMA2_70B, "M": (1, 16, 64, 256, 1024, 4096),
                             "abits": (6, 8)},
}
