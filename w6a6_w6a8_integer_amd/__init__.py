"""MI355X (gfx950) W6A6 / W6A8 group-quantized linear layer (the FlexQ hot path).

A thin ctypes binding over ``libflexq.so`` (C ABI in ``include/flexq.h``).  This
module only marshals arguments: it takes torch CUDA tensors for device memory,
passes their pointers and the current HIP stream, and allocates outputs when the
caller does not supply them.  Every step of the computation runs in the HIP
kernels; if the library is missing the calls raise instead of falling back.

Entry points (same names as the C ABI):

* :func:`pack_w6`        fp16 W[N][K] -> packed 6-bit codes + fp16 group scales
* :func:`quant_act`      fp16 X[M][K] -> int8 codes (INT6 or INT8 range) + fp32 scales
* :func:`gemm_w6ax`      Y[M][N] fp16 = sum over groups of int32 dot x s_w x s_a
* :func:`linear_w6ax`    Y[M][N] fp16 from fp16 X in one call (both kernels, q_a / s_a
  in a caller-supplied or binding-allocated workspace)
* :func:`gemm_w6ax_splitk` the GEMM with K split over workgroups (mid-sized M),
  fp32 partials summed in a fixed order
* :func:`gemm_w6ax_group_dots`  the int32 group dots (verification)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflexq.so")

GROUP = 128
DECODE_MAX_M = 64
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
# the prefill kernel with a fixed workgroup tile (rows x columns)
PATH_PREFILL_256X128, PATH_PREFILL_128X128, PATH_PREFILL_128X64 = 3, 4, 5
# 256 x 128 tiles from 4 MFMA waves with 4 loader waves staging the operands
PATH_PREFILL_256X128_WS = 6
# the prefill kernel with 64 x 128 tiles (few tokens on wide layers)
PATH_PREFILL_64X128 = 7

STATUS_NAMES = {0: "FLEXQ_SUCCESS", 1: "FLEXQ_ERROR_INVALID_VALUE", 2: "FLEXQ_ERROR_UNSUPPORTED",
                3: "FLEXQ_ERROR_LAUNCH"}

# (restype, argtypes) of every symbol include/flexq.h declares
_P, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
SIGNATURES = {
    "flexq_abi_version": (ctypes.c_int, []),
    "flexq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "flexq_packed_w6_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "flexq_pack_w6": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "flexq_quant_act": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _P, _P]),
    "flexq_packed_a6_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "flexq_quant_act_a6_packed": (ctypes.c_int, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "flexq_gemm_w6a6_packed": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _P]),
    "flexq_blocked_act_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "flexq_quant_act_blocked": (ctypes.c_int, [_P, _I64, _I64, _I32, _I32, _P, _P, _P]),
    "flexq_gemm_w6ax_blocked": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P,
                                               _P]),
    "flexq_gemm_w6ax": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    "flexq_gemm_w6ax_path": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32,
                                            _P, _P]),
    "flexq_gemm_w6ax_group_dots": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _P, _P]),
    "flexq_gemm_w6ax_auto_path": (ctypes.c_int, [_I64, _I64, _I64]),
    "flexq_gemm_w6ax_prefill_tile": (ctypes.c_int, [_I64, _I64, _I64]),
    "flexq_gemm_w6ax_prefill_main_cols": (ctypes.c_int64, [_I64, _I64, _I64]),
    "flexq_gemm_w6ax_splitk": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32,
                                              _I32, _I32, _P, ctypes.c_size_t, _P, _P, _P]),
    "flexq_gemm_w6ax_splitk_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I32]),
    "flexq_gemm_w6ax_splitk_plan": (ctypes.c_int32, [_I64, _I64, _I64, _P]),
    "flexq_linear_w6ax_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "flexq_linear_w6ax": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P,
                                         ctypes.c_size_t, _P, _P]),
    "flexq_linear_w6ax_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P,
                                                 _P]),
}
# the on-device peak measurements of include/flexq_peaks.h
PEAK_SIGNATURES = {
    "flexq_peak_sink_bytes": (ctypes.c_size_t, []),
    "flexq_peak_hbm_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "flexq_peak_mfma_i8": (ctypes.c_int, [_I64, _I32, _P, _P, _P]),
    "flexq_peak_mfma_i8_workgroups": (ctypes.c_int64, []),
    "flexq_peak_mfma_i8_rescale": (ctypes.c_int, [_I64, _P, _P, _P]),
    "flexq_peak_mfma_i8_rescale_waves": (ctypes.c_int64, []),
}
# bytes of the library's per-GPU staging array behind flexq_linear_w6ax_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class FlexqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = lib().flexq_status_string(status).decode()
        super().__init__(f"{where}: {text}")


def lib():
    """The loaded libflexq.so (ctypes), with argument types set."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(there is no CPU fallback)")
        h = ctypes.CDLL(LIB_PATH)  # after `import torch`, so the HIP runtime is shared
        for name, (res, args) in {**SIGNATURES, **PEAK_SIGNATURES}.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise FlexqError(status, where)


def _stream(t: torch.Tensor | None = None) -> int:
    dev = t.device if t is not None else None
    return torch.cuda.current_stream(dev).cuda_stream


def _tensor(t, dtype, name: str, shape=None, min_bytes=None):
    """Check one tensor argument before anything reaches the C ABI, which sees only
    pointers and cannot tell a wrong buffer from a right one: type, dtype, exact
    shape (or a minimum size for flat buffers) and contiguity.  Where the tensors
    live is checked once for all of them (_on_gpu), after every shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; "
                         f"at least {min_bytes} are needed")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(**tensors):
    """Every argument is a CUDA (HIP) tensor, all on one device; returns it."""
    dev = None
    for name, t in tensors.items():
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")
    return dev


def _matrix(t, dtype, name: str):
    """A 2-D tensor argument whose shape defines the problem size."""
    if isinstance(t, torch.Tensor) and t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return _tensor(t, dtype, name)


def _groups(K: int, name: str) -> int:
    if K <= 0 or K % GROUP:
        raise ValueError(f"{name}: K = {K} must be a positive multiple of {GROUP}")
    return K // GROUP


def _cols(N: int) -> int:
    N = int(N)
    if N < 0 or N % 16:
        raise ValueError(f"N = {N} must be a non-negative multiple of 16")
    return N


def _packed(w_packed, N: int, K: int):
    """Packed weights: a flat int32 buffer of at least 0.75 * N * K bytes."""
    if isinstance(w_packed, torch.Tensor) and w_packed.dim() != 1:
        raise ValueError(f"w_packed must be 1-D, got shape {tuple(w_packed.shape)}")
    return _tensor(w_packed, torch.int32, "w_packed", min_bytes=3 * N * K // 4)


def packed_w6_bytes(N: int, K: int) -> int:
    return int(lib().flexq_packed_w6_bytes(N, K))


def packed_w6_words(N: int, K: int) -> int:
    return packed_w6_bytes(N, K) // 4


def pack_w6(w: torch.Tensor, w_packed: torch.Tensor | None = None,
            s_w: torch.Tensor | None = None):
    """fp16 W[N][K] -> (w_packed int32[3*N*K/16] holding the packed dwords,
    s_w fp16[K/128][N], group-major)."""
    _matrix(w, torch.float16, "w")
    N, K = w.shape
    G = _groups(K, "pack_w6")
    _cols(N)
    if w_packed is None:
        w_packed = torch.empty(max(1, 3 * N * K // 16), dtype=torch.int32, device=w.device)
    if s_w is None:
        s_w = torch.empty((G, N), dtype=torch.float16, device=w.device)
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    _on_gpu(w=w, w_packed=w_packed, s_w=s_w)
    _check(lib().flexq_pack_w6(w.data_ptr(), N, K, GROUP, w_packed.data_ptr(), s_w.data_ptr(),
                               _stream(w)), "flexq_pack_w6")
    return w_packed, s_w


def quant_act(x: torch.Tensor, abits: int, q_a: torch.Tensor | None = None,
              s_a: torch.Tensor | None = None):
    """fp16 X[M][K] -> (q_a int8[M][K], s_a fp32[K/128][M], group-major); abits 6 or 8."""
    _matrix(x, torch.float16, "x")
    M, K = x.shape
    G = _groups(K, "quant_act")
    if q_a is None:
        q_a = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((G, M), dtype=torch.float32, device=x.device)
    _tensor(q_a, torch.int8, "q_a", shape=(M, K))
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _on_gpu(x=x, q_a=q_a, s_a=s_a)
    _check(lib().flexq_quant_act(x.data_ptr(), M, K, GROUP, abits, q_a.data_ptr(),
                                 s_a.data_ptr(), _stream(x)), "flexq_quant_act")
    return q_a, s_a


def packed_a6_bytes(M: int, K: int) -> int:
    return int(lib().flexq_packed_a6_bytes(M, K))


def quant_act_a6_packed(x: torch.Tensor, q_a6p: torch.Tensor | None = None,
                        s_a: torch.Tensor | None = None):
    """fp16 X[M][K] -> (q_a6p int32[M][3*K/16]: the A6 codes packed 16 per 3 dwords,
    s_a fp32[K/128][M]); the codes and scales of quant_act(x, 6)."""
    _matrix(x, torch.float16, "x")
    M, K = x.shape
    G = _groups(K, "quant_act_a6_packed")
    if q_a6p is None:
        q_a6p = torch.empty((M, 3 * K // 16), dtype=torch.int32, device=x.device)
    if s_a is None:
        s_a = torch.empty((G, M), dtype=torch.float32, device=x.device)
    _tensor(q_a6p, torch.int32, "q_a6p", shape=(M, 3 * K // 16))
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _on_gpu(x=x, q_a6p=q_a6p, s_a=s_a)
    _check(lib().flexq_quant_act_a6_packed(x.data_ptr(), M, K, GROUP, q_a6p.data_ptr(),
                                           s_a.data_ptr(), _stream(x)),
           "flexq_quant_act_a6_packed")
    return q_a6p, s_a


def gemm_w6a6_packed(q_a6p: torch.Tensor, s_a: torch.Tensor, w_packed: torch.Tensor,
                     s_w: torch.Tensor, N: int, y: torch.Tensor | None = None):
    """Y fp16[M][N] from packed A6 activations (q_a6p int32[M][3*K/16], s_a
    fp32[K/128][M]) and packed weights: the weight-streaming kernel, the bits of
    gemm_w6ax on the unpacked codes."""
    _matrix(q_a6p, torch.int32, "q_a6p")
    M, words = q_a6p.shape
    if words % 3:
        raise ValueError(f"q_a6p has {words} dwords per row; a multiple of 3 is needed")
    K = words // 3 * 16
    G = _groups(K, "gemm_w6a6_packed")
    N = _cols(N)
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=q_a6p.device)
    _tensor(y, torch.float16, "y", shape=(M, N))
    _on_gpu(q_a6p=q_a6p, s_a=s_a, w_packed=w_packed, s_w=s_w, y=y)
    _check(lib().flexq_gemm_w6a6_packed(q_a6p.data_ptr(), s_a.data_ptr(), w_packed.data_ptr(),
                                        s_w.data_ptr(), M, N, K, GROUP, y.data_ptr(),
                                        _stream(q_a6p)), "flexq_gemm_w6a6_packed")
    return y


def blocked_act_bytes(M: int, K: int) -> int:
    return int(lib().flexq_blocked_act_bytes(M, K))


def quant_act_blocked(x: torch.Tensor, abits: int, q_a_blk: torch.Tensor | None = None,
                      s_a: torch.Tensor | None = None):
    """fp16 X[M][K] -> (q_a_blk int8[ceil(M/16)*16*K]: the codes in 16-row blocks, the
    order the streaming GEMM feeds its MFMAs, s_a fp32[K/128][M]); the codes and
    scales of quant_act(x, abits)."""
    _matrix(x, torch.float16, "x")
    M, K = x.shape
    G = _groups(K, "quant_act_blocked")
    nbytes = (M + 15) // 16 * 16 * K
    if q_a_blk is None:
        q_a_blk = torch.empty(max(1, nbytes), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((G, M), dtype=torch.float32, device=x.device)
    if isinstance(q_a_blk, torch.Tensor) and q_a_blk.dim() != 1:
        raise ValueError(f"q_a_blk must be 1-D, got shape {tuple(q_a_blk.shape)}")
    _tensor(q_a_blk, torch.int8, "q_a_blk", min_bytes=nbytes)
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _on_gpu(x=x, q_a_blk=q_a_blk, s_a=s_a)
    _check(lib().flexq_quant_act_blocked(x.data_ptr(), M, K, GROUP, abits, q_a_blk.data_ptr(),
                                         s_a.data_ptr(), _stream(x)), "flexq_quant_act_blocked")
    return q_a_blk, s_a


def gemm_w6ax_blocked(q_a_blk: torch.Tensor, s_a: torch.Tensor, w_packed: torch.Tensor,
                      s_w: torch.Tensor, N: int, abits: int, y: torch.Tensor | None = None):
    """Y fp16[M][N] from blocked activation codes (q_a_blk, from quant_act_blocked; M and
    K come from s_a fp32[K/128][M]) and packed weights: the streaming kernel, the bits of
    gemm_w6ax on the row-major codes."""
    _matrix(s_a, torch.float32, "s_a")
    G, M = s_a.shape
    K = G * GROUP
    N = _cols(N)
    if isinstance(q_a_blk, torch.Tensor) and q_a_blk.dim() != 1:
        raise ValueError(f"q_a_blk must be 1-D, got shape {tuple(q_a_blk.shape)}")
    _tensor(q_a_blk, torch.int8, "q_a_blk", min_bytes=(M + 15) // 16 * 16 * K)
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=s_a.device)
    _tensor(y, torch.float16, "y", shape=(M, N))
    _on_gpu(q_a_blk=q_a_blk, s_a=s_a, w_packed=w_packed, s_w=s_w, y=y)
    _check(lib().flexq_gemm_w6ax_blocked(q_a_blk.data_ptr(), s_a.data_ptr(), w_packed.data_ptr(),
                                         s_w.data_ptr(), M, N, K, GROUP, abits, y.data_ptr(),
                                         _stream(s_a)), "flexq_gemm_w6ax_blocked")
    return y


def gemm_w6ax(q_a: torch.Tensor, s_a: torch.Tensor, w_packed: torch.Tensor, s_w: torch.Tensor,
              N: int, abits: int, y: torch.Tensor | None = None, path: int = PATH_AUTO):
    """Y fp16[M][N] from quantized activations (q_a int8[M][K], s_a fp32[K/128][M])
    and packed weights (w_packed, s_w fp16[K/128][N])."""
    _matrix(q_a, torch.int8, "q_a")
    M, K = q_a.shape
    G = _groups(K, "gemm_w6ax")
    N = _cols(N)
    dev = q_a.device
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _tensor(y, torch.float16, "y", shape=(M, N))
    _on_gpu(q_a=q_a, s_a=s_a, w_packed=w_packed, s_w=s_w, y=y)
    _check(lib().flexq_gemm_w6ax_path(q_a.data_ptr(), s_a.data_ptr(), w_packed.data_ptr(),
                                      s_w.data_ptr(), M, N, K, GROUP, abits, path, y.data_ptr(),
                                      _stream(q_a)), "flexq_gemm_w6ax")
    return y


def splitk_plan(M: int, N: int, K: int) -> tuple[int, int]:
    """(S, tile path) that gemm_w6ax_splitk takes for this shape on the current
    device when asked to choose (flexq_gemm_w6ax_splitk_plan)."""
    tile = ctypes.c_int32(0)
    S = int(lib().flexq_gemm_w6ax_splitk_plan(M, N, K, ctypes.byref(tile)))
    return S, int(tile.value)


def splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    return int(lib().flexq_gemm_w6ax_splitk_workspace_bytes(M, N, K, splits))


def gemm_w6ax_splitk(q_a: torch.Tensor, s_a: torch.Tensor, w_packed: torch.Tensor,
                     s_w: torch.Tensor, N: int, abits: int, splits: int = 0,
                     path: int = PATH_PREFILL, y: torch.Tensor | None = None,
                     acc: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Split-K GEMM (flexq_gemm_w6ax_splitk): Y fp16[M][N] with K cut into `splits`
    slices (0 = the planned count) whose fp32 partials are summed in ascending order;
    `acc` (fp32[M][N], optional) receives the fp32 sums.  The workspace (uint8, at
    least splitk_workspace_bytes(M, N, K, splits)) is allocated here when not passed."""
    _matrix(q_a, torch.int8, "q_a")
    M, K = q_a.shape
    G = _groups(K, "gemm_w6ax_splitk")
    N = _cols(N)
    dev = q_a.device
    _tensor(s_a, torch.float32, "s_a", shape=(G, M))
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _tensor(y, torch.float16, "y", shape=(M, N))
    if acc is not None:
        _tensor(acc, torch.float32, "acc", shape=(M, N))
    need = splitk_workspace_bytes(M, N, K, splits)
    if workspace is None:
        workspace = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    if isinstance(workspace, torch.Tensor) and workspace.dim() != 1:
        raise ValueError(f"workspace must be 1-D, got shape {tuple(workspace.shape)}")
    _tensor(workspace, torch.uint8, "workspace", min_bytes=need)
    tensors = dict(q_a=q_a, s_a=s_a, w_packed=w_packed, s_w=s_w, y=y, workspace=workspace)
    if acc is not None:
        tensors["acc"] = acc
    _on_gpu(**tensors)
    _check(lib().flexq_gemm_w6ax_splitk(q_a.data_ptr(), s_a.data_ptr(), w_packed.data_ptr(),
                                        s_w.data_ptr(), M, N, K, GROUP, abits, path, splits,
                                        workspace.data_ptr(), workspace.numel(), y.data_ptr(),
                                        acc.data_ptr() if acc is not None else None,
                                        _stream(q_a)), "flexq_gemm_w6ax_splitk")
    return y


def linear_w6ax_workspace_bytes(M: int, K: int) -> int:
    return int(lib().flexq_linear_w6ax_workspace_bytes(M, K))


def linear_w6ax(x: torch.Tensor, w_packed: torch.Tensor, s_w: torch.Tensor, N: int, abits: int,
                y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Y fp16[M][N] from fp16 X[M][K] and packed weights (flexq_linear_w6ax); the
    workspace (uint8, at least linear_w6ax_workspace_bytes(M, K)) is allocated here
    when the caller does not pass one."""
    _matrix(x, torch.float16, "x")
    M, K = x.shape
    G = _groups(K, "linear_w6ax")
    N = _cols(N)
    dev = x.device
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _tensor(y, torch.float16, "y", shape=(M, N))
    need = linear_w6ax_workspace_bytes(M, K)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    if isinstance(workspace, torch.Tensor) and workspace.dim() != 1:
        raise ValueError(f"workspace must be 1-D, got shape {tuple(workspace.shape)}")
    _tensor(workspace, torch.uint8, "workspace", min_bytes=need)
    _on_gpu(x=x, w_packed=w_packed, s_w=s_w, y=y, workspace=workspace)
    _check(lib().flexq_linear_w6ax(x.data_ptr(), w_packed.data_ptr(), s_w.data_ptr(), M, N, K,
                                   GROUP, abits, workspace.data_ptr(), workspace.numel(),
                                   y.data_ptr(), _stream(x)), "flexq_linear_w6ax")
    return y


def linear_w6ax_noalloc(x: torch.Tensor, w_packed: torch.Tensor, s_w: torch.Tensor, N: int,
                        abits: int, y: torch.Tensor) -> torch.Tensor:
    """flexq_linear_w6ax_noalloc: the one-call layer with its activation codes staged
    in the library's own per-GPU device array, for callers that cannot allocate; the
    caller passes the output.  Calls that may overlap in time on one GPU race on
    that array (calls ordered on one stream are safe)."""
    _matrix(x, torch.float16, "x")
    M, K = x.shape
    G = _groups(K, "linear_w6ax_noalloc")
    N = _cols(N)
    _packed(w_packed, N, K)
    _tensor(s_w, torch.float16, "s_w", shape=(G, N))
    _tensor(y, torch.float16, "y", shape=(M, N))
    _on_gpu(x=x, w_packed=w_packed, s_w=s_w, y=y)
    _check(lib().flexq_linear_w6ax_noalloc(x.data_ptr(), w_packed.data_ptr(), s_w.data_ptr(), M,
                                           N, K, GROUP, abits, y.data_ptr(), _stream(x)),
           "flexq_linear_w6ax_noalloc")
    return y


def gemm_w6ax_group_dots(q_a: torch.Tensor, w_packed: torch.Tensor, N: int,
                         dots: torch.Tensor | None = None):
    """int32 d[M][N][K/128] through the production unpack + int8 MFMA."""
    _matrix(q_a, torch.int8, "q_a")
    M, K = q_a.shape
    G = _groups(K, "gemm_w6ax_group_dots")
    N = _cols(N)
    dev = q_a.device
    _packed(w_packed, N, K)
    if dots is None:
        dots = torch.empty((M, N, G), dtype=torch.int32, device=dev)
    _tensor(dots, torch.int32, "dots", shape=(M, N, G))
    _on_gpu(q_a=q_a, w_packed=w_packed, dots=dots)
    _check(lib().flexq_gemm_w6ax_group_dots(q_a.data_ptr(), w_packed.data_ptr(), M, N, K, GROUP,
                                            dots.data_ptr(), _stream(q_a)),
           "flexq_gemm_w6ax_group_dots")
    return dots


def peak_hbm_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Enqueue flexq_peak_hbm_read over all of `buf` (a contiguous CUDA tensor whose
    size is a multiple of 16 bytes); `sink`: uint8 CUDA tensor of peak_sink_bytes()."""
    _tensor(sink, torch.uint8, "sink", min_bytes=peak_sink_bytes())
    _on_gpu(buf=buf, sink=sink)
    rc = lib().flexq_peak_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                   sink.data_ptr(), _stream(buf))
    if rc != 0:
        raise RuntimeError(f"flexq_peak_hbm_read returned {rc}")


def peak_mfma_i8(iters: int, valu_per_mfma: int, sink: torch.Tensor,
                 clock: torch.Tensor) -> int:
    """Enqueue flexq_peak_mfma_i8; returns the integer ops the launch performs.
    clock: int64 CUDA tensor of 2 (shader cycles, 100 MHz ticks of wave 0)."""
    _tensor(sink, torch.uint8, "sink", min_bytes=peak_sink_bytes())
    _tensor(clock, torch.int64, "clock", shape=(2,))
    _on_gpu(sink=sink, clock=clock)
    rc = lib().flexq_peak_mfma_i8(iters, valu_per_mfma, sink.data_ptr(), clock.data_ptr(),
                                  _stream(sink))
    if rc != 0:
        raise RuntimeError(f"flexq_peak_mfma_i8 returned {rc}")
    return 2 * 32768 * 4 * iters * 4 * int(lib().flexq_peak_mfma_i8_workgroups())


def peak_mfma_i8_rescale(iters: int, sink: torch.Tensor, clock: torch.Tensor) -> int:
    """Enqueue flexq_peak_mfma_i8_rescale (int8 MFMA chains with the exact group
    rescale, LDS operand reads and a barrier per group); returns the integer ops."""
    _tensor(sink, torch.uint8, "sink", min_bytes=peak_sink_bytes())
    _tensor(clock, torch.int64, "clock", shape=(2,))
    _on_gpu(sink=sink, clock=clock)
    rc = lib().flexq_peak_mfma_i8_rescale(iters, sink.data_ptr(), clock.data_ptr(), _stream(sink))
    if rc != 0:
        raise RuntimeError(f"flexq_peak_mfma_i8_rescale returned {rc}")
    return 2 * 32768 * 16 * iters * int(lib().flexq_peak_mfma_i8_rescale_waves())


def peak_sink_bytes() -> int:
    return int(lib().flexq_peak_sink_bytes())


def prefill_tile(M: int, N: int, K: int) -> int:
    """PATH_PREFILL_256X128 / _128X128 / _128X64: the tile PATH_PREFILL uses for this
    shape on the current device (flexq_gemm_w6ax_prefill_tile)."""
    return int(lib().flexq_gemm_w6ax_prefill_tile(M, N, K))


def prefill_main_cols(M: int, N: int, K: int) -> int:
    """Columns the first PATH_PREFILL launch covers on the current device; N unless
    a second launch of 128 x 64 tiles takes the rest (flexq_gemm_w6ax_prefill_main_cols)."""
    return int(lib().flexq_gemm_w6ax_prefill_main_cols(M, N, K))


def auto_path(M: int, N: int, K: int) -> int:
    """PATH_DECODE or PATH_PREFILL: the kernel PATH_AUTO runs for this shape on the
    current device (flexq_gemm_w6ax_auto_path)."""
    return int(lib().flexq_gemm_w6ax_auto_path(M, N, K))


class W6AxLinear:
    """A quantized nn.Linear-shaped layer: packed 6-bit weights resident in HBM,
    activation quantization fused in front of every product (A6 or A8)."""

    def __init__(self, weight_fp16: torch.Tensor, abits: int = 6):
        self.N, self.K = weight_fp16.shape
        self.abits = abits
        self.w_packed, self.s_w = pack_w6(weight_fp16.contiguous())

    def __call__(self, x_fp16: torch.Tensor, path: int = PATH_AUTO) -> torch.Tensor:
        if path == PATH_AUTO:
            return linear_w6ax(x_fp16.contiguous(), self.w_packed, self.s_w, self.N, self.abits)
        q_a, s_a = quant_act(x_fp16.contiguous(), self.abits)
        return gemm_w6ax(q_a, s_a, self.w_packed, self.s_w, self.N, self.abits, path=path)
