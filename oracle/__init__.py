"""Python front end of the plain CPU oracle (``flexq_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The GPU library never
calls it and shares no code with it.

Every function takes and returns numpy arrays.  fp16 tensors are passed as
numpy ``float16`` arrays (their bits are what the oracle reads).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libflexq_oracle.so")
_lib = None
GROUP = 128

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc: strict IEEE binary32, no contraction."""
    src = os.path.join(_HERE, "flexq_oracle.c")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", src, "-o", _LIB_PATH + ".tmp", "-lm"]
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
    sig = {
        "oracle_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_quant_w6": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
        "oracle_pack_unit": (None, [_P, _P]),
        "oracle_unpack_unit": (None, [_P, _P]),
        "oracle_unit_offset": (_I64, [_I64, _I64, _I64]),
        "oracle_pack_codes": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_unpack_codes": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_pack_w6": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P]),
        "oracle_quant_act": (ctypes.c_int, [_P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
        "oracle_pack_act_a6": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_unpack_act_a6": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_block_act": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_unblock_act": (ctypes.c_int, [_P, _I64, _I64, _P]),
        "oracle_group_dots": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I64, _P, ctypes.c_int]),
        "oracle_gemm": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P,
                                       ctypes.c_int]),
        "oracle_gemm_packed": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P,
                                              _P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _threads(nthreads):
    if nthreads is not None:
        return int(nthreads)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (rc={rc})")


# --- scalar helpers ---------------------------------------------------------

def f16_to_f32(bits: int) -> float:
    return float(_load().oracle_f16_to_f32(int(bits)))


def f32_to_f16(value: float) -> int:
    return int(_load().oracle_f32_to_f16(float(np.float32(value))))


# --- weights ----------------------------------------------------------------

def quant_w6(w: np.ndarray, group: int = GROUP):
    """w fp16 [N][K] -> (qw int8 [N][K], sw fp16 [N][K/group])."""
    w = _c(w, np.float16)
    N, K = w.shape
    qw = np.empty((N, K), np.int8)
    sw = np.empty((N, K // group), np.float16)
    _check(_load().oracle_quant_w6(w.ctypes.data, N, K, group, qw.ctypes.data, sw.ctypes.data),
           "quant_w6")
    return qw, sw


def pack_unit(q) -> np.ndarray:
    q = _c(np.asarray(q, dtype=np.int8), np.int8)
    assert q.shape == (16,)
    d = np.zeros(3, np.uint32)
    _load().oracle_pack_unit(q.ctypes.data, d.ctypes.data)
    return d


def unpack_unit(d) -> np.ndarray:
    d = _c(np.asarray(d, dtype=np.uint32), np.uint32)
    assert d.shape == (3,)
    q = np.zeros(16, np.int8)
    _load().oracle_unpack_unit(d.ctypes.data, q.ctypes.data)
    return q


def unit_offset(n: int, u: int, K: int) -> int:
    return int(_load().oracle_unit_offset(n, u, K))


def packed_words(N: int, K: int) -> int:
    return 3 * N * K // 16


def pack_codes(qw: np.ndarray) -> np.ndarray:
    qw = _c(qw, np.int8)
    N, K = qw.shape
    wp = np.zeros(packed_words(N, K), np.uint32)
    _check(_load().oracle_pack_codes(qw.ctypes.data, N, K, wp.ctypes.data), "pack_codes")
    return wp


def unpack_codes(wp: np.ndarray, N: int, K: int) -> np.ndarray:
    wp = _c(wp, np.uint32)
    assert wp.size == packed_words(N, K)
    qw = np.empty((N, K), np.int8)
    _check(_load().oracle_unpack_codes(wp.ctypes.data, N, K, qw.ctypes.data), "unpack_codes")
    return qw


def pack_w6(w: np.ndarray, group: int = GROUP):
    """w fp16 [N][K] -> (wp uint32 [3*N*K/16], sw fp16 [N][K/group])."""
    w = _c(w, np.float16)
    N, K = w.shape
    wp = np.zeros(packed_words(N, K), np.uint32)
    sw = np.empty((N, K // group), np.float16)
    _check(_load().oracle_pack_w6(w.ctypes.data, N, K, group, wp.ctypes.data, sw.ctypes.data),
           "pack_w6")
    return wp, sw


# --- activations --------------------------------------------------------------

def quant_act(x: np.ndarray, abits: int, group: int = GROUP):
    """x fp16 [M][K] -> (qa int8 [M][K], sa fp32 [M][K/group])."""
    x = _c(x, np.float16)
    M, K = x.shape
    qa = np.empty((M, K), np.int8)
    sa = np.empty((M, K // group), np.float32)
    _check(_load().oracle_quant_act(x.ctypes.data, M, K, group, abits, qa.ctypes.data,
                                    sa.ctypes.data), "quant_act")
    return qa, sa


def pack_act_a6(qa: np.ndarray) -> np.ndarray:
    """Codes qa int8 [M][K] (each in [-32, 31]) -> uint32 [M][3*K/16]: 16 codes per
    3-dword unit (the packed-weight unit), the units of a row in order."""
    qa = _c(qa, np.int8)
    M, K = qa.shape
    qp = np.zeros((M, 3 * K // 16), np.uint32)
    _check(_load().oracle_pack_act_a6(qa.ctypes.data, M, K, qp.ctypes.data), "pack_act_a6")
    return qp


def block_act(qa: np.ndarray) -> np.ndarray:
    """Codes qa int8 [M][K] -> int8 [ceil(M/16)*16*K] in 16-row blocks: block b, group
    g, 64-deep half h, row r, byte c at b*16*K + g*2048 + h*1024 + r*64 + c (pad rows
    hold zero codes)."""
    qa = _c(qa, np.int8)
    M, K = qa.shape
    out = np.empty((M + 15) // 16 * 16 * K, np.int8)
    _check(_load().oracle_block_act(qa.ctypes.data, M, K, out.ctypes.data), "block_act")
    return out


def unblock_act(blk: np.ndarray, M: int, K: int) -> np.ndarray:
    blk = _c(blk, np.int8)
    assert blk.size == (M + 15) // 16 * 16 * K
    qa = np.empty((M, K), np.int8)
    _check(_load().oracle_unblock_act(blk.ctypes.data, M, K, qa.ctypes.data), "unblock_act")
    return qa


def unpack_act_a6(qp: np.ndarray, K: int) -> np.ndarray:
    """uint32 [M][3*K/16] -> codes int8 [M][K]."""
    qp = _c(qp, np.uint32)
    M = qp.shape[0]
    assert qp.shape == (M, 3 * K // 16)
    qa = np.empty((M, K), np.int8)
    _check(_load().oracle_unpack_act_a6(qp.ctypes.data, M, K, qa.ctypes.data), "unpack_act_a6")
    return qa


# --- products -----------------------------------------------------------------

def group_dots(qa: np.ndarray, qw: np.ndarray, group: int = GROUP, nthreads=None):
    """int32 [M][N][K/group]."""
    qa = _c(qa, np.int8)
    qw = _c(qw, np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    dots = np.empty((M, N, K // group), np.int32)
    _check(_load().oracle_group_dots(qa.ctypes.data, qw.ctypes.data, M, N, K, group,
                                     dots.ctypes.data, _threads(nthreads)), "group_dots")
    return dots


def gemm(qa, sa, qw, sw, group: int = GROUP, nthreads=None, want_acc: bool = False):
    """Y fp16 [M][N]; with want_acc also (acc fp32 [M][N], S float64 [M][N])."""
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float16)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.empty((M, N), np.float16)
    acc = np.empty((M, N), np.float32) if want_acc else None
    S = np.empty((M, N), np.float64) if want_acc else None
    _check(_load().oracle_gemm(qa.ctypes.data, sa.ctypes.data, qw.ctypes.data, sw.ctypes.data,
                               M, N, K, group, y.ctypes.data,
                               acc.ctypes.data if want_acc else None,
                               S.ctypes.data if want_acc else None, _threads(nthreads)), "gemm")
    return (y, acc, S) if want_acc else y


def gemm_packed(qa, sa, wp, sw, N: int, group: int = GROUP, nthreads=None,
                want_acc: bool = False):
    """Same as :func:`gemm` but from the packed weights."""
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    wp = _c(wp, np.uint32)
    sw = _c(sw, np.float16)
    M, K = qa.shape
    y = np.empty((M, N), np.float16)
    acc = np.empty((M, N), np.float32) if want_acc else None
    S = np.empty((M, N), np.float64) if want_acc else None
    _check(_load().oracle_gemm_packed(qa.ctypes.data, sa.ctypes.data, wp.ctypes.data,
                                      sw.ctypes.data, M, N, K, group, y.ctypes.data,
                                      acc.ctypes.data if want_acc else None,
                                      S.ctypes.data if want_acc else None, _threads(nthreads)),
           "gemm_packed")
    return (y, acc, S) if want_acc else y
