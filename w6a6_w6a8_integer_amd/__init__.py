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
    "flexq_gemm_w6ax": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    "flexq_gemm_w6ax_path": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32,
                                            _P, _P]),
    "flexq_gemm_w6ax_group_dots": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _P, _P]),
    "flexq_gemm_w6ax_auto_path": (ctypes.c_int, [_I64, _I64, _I64]),
    "flexq_gemm_w6ax_prefill_tile": (ctypes.c_int, [_I64, _I64, _I64]),
    "flexq_gemm_w6ax_prefill_main_cols": (ctypes.c_int64, [_I64, _I64, _I64]),
    "flexq_linear_w6ax_workspace_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "flexq_linear_w6ax": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P,
                                         ctypes.c_size_t, _P, _P]),
}

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
        for name, (res, args) in SIGNATURES.items():
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


def _cuda(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def packed_w6_bytes(N: int, K: int) -> int:
    return int(lib().flexq_packed_w6_bytes(N, K))


def packed_w6_words(N: int, K: int) -> int:
    return packed_w6_bytes(N, K) // 4


def pack_w6(w: torch.Tensor, w_packed: torch.Tensor | None = None,
            s_w: torch.Tensor | None = None):
    """fp16 W[N][K] -> (w_packed int32[3*N*K/16] holding the packed dwords,
    s_w fp16[K/128][N], group-major)."""
    _cuda(w, torch.float16, "w")
    N, K = w.shape
    if w_packed is None:
        w_packed = torch.empty(max(1, packed_w6_words(N, K)), dtype=torch.int32, device=w.device)
    if s_w is None:
        s_w = torch.empty((K // GROUP, N), dtype=torch.float16, device=w.device)
    _check(lib().flexq_pack_w6(w.data_ptr(), N, K, GROUP, w_packed.data_ptr(), s_w.data_ptr(),
                               _stream(w)), "flexq_pack_w6")
    return w_packed, s_w


def quant_act(x: torch.Tensor, abits: int, q_a: torch.Tensor | None = None,
              s_a: torch.Tensor | None = None):
    """fp16 X[M][K] -> (q_a int8[M][K], s_a fp32[K/128][M], group-major); abits 6 or 8."""
    _cuda(x, torch.float16, "x")
    M, K = x.shape
    if q_a is None:
        q_a = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((K // GROUP, M), dtype=torch.float32, device=x.device)
    _check(lib().flexq_quant_act(x.data_ptr(), M, K, GROUP, abits, q_a.data_ptr(),
                                 s_a.data_ptr(), _stream(x)), "flexq_quant_act")
    return q_a, s_a


def gemm_w6ax(q_a: torch.Tensor, s_a: torch.Tensor, w_packed: torch.Tensor, s_w: torch.Tensor,
              N: int, abits: int, y: torch.Tensor | None = None, path: int = PATH_AUTO):
    """Y fp16[M][N] from quantized activations and packed weights."""
    _cuda(q_a, torch.int8, "q_a")
    M, K = q_a.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=q_a.device)
    _check(lib().flexq_gemm_w6ax_path(q_a.data_ptr(), s_a.data_ptr(), w_packed.data_ptr(),
                                      s_w.data_ptr(), M, N, K, GROUP, abits, path, y.data_ptr(),
                                      _stream(q_a)), "flexq_gemm_w6ax")
    return y


def linear_w6ax_workspace_bytes(M: int, K: int) -> int:
    return int(lib().flexq_linear_w6ax_workspace_bytes(M, K))


def linear_w6ax(x: torch.Tensor, w_packed: torch.Tensor, s_w: torch.Tensor, N: int, abits: int,
                y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Y fp16[M][N] from fp16 X[M][K] and packed weights (flexq_linear_w6ax); the
    workspace (uint8, at least linear_w6ax_workspace_bytes(M, K)) is allocated here
    when the caller does not pass one."""
    _cuda(x, torch.float16, "x")
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(1, linear_w6ax_workspace_bytes(M, K)), dtype=torch.uint8,
                                device=x.device)
    ws_ptr = workspace.data_ptr()
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().flexq_linear_w6ax(x.data_ptr(), w_packed.data_ptr(), s_w.data_ptr(), M, N, K,
                                   GROUP, abits, ws_ptr, ws_bytes, y.data_ptr(), _stream(x)),
           "flexq_linear_w6ax")
    return y


def gemm_w6ax_group_dots(q_a: torch.Tensor, w_packed: torch.Tensor, N: int,
                         dots: torch.Tensor | None = None):
    """int32 d[M][N][K/128] through the production unpack + int8 MFMA."""
    _cuda(q_a, torch.int8, "q_a")
    M, K = q_a.shape
    if dots is None:
        dots = torch.empty((M, N, K // GROUP), dtype=torch.int32, device=q_a.device)
    _check(lib().flexq_gemm_w6ax_group_dots(q_a.data_ptr(), w_packed.data_ptr(), M, N, K, GROUP,
                                            dots.data_ptr(), _stream(q_a)),
           "flexq_gemm_w6ax_group_dots")
    return dots


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
