"""The Y tolerance for results whose fp32 summation order differs from the sequential
definition (the split-K GEMM), as the FlexQ blog leaves the order open: its
"Bridging Software and Hardware with BTC" section fixes exact integer group products
and a dequantization fused into the GEMM, not an order of the fp32 additions.

An output passes when |Y_gpu - Y_ref| <= one fp16 ulp of Y_ref, or, where the two
differ by more (an fp32 sum that lands near an fp16 rounding boundary), when the
fp32 sum the GPU rounded satisfies |acc_gpu - acc_ref| <= 1e-5 * S with
S = sum over groups of |t * s_a|, the magnitude of the terms summed (a relative
bound on the sum of magnitudes stays meaningful where the terms cancel).
"""
import numpy as np

REL = 1e-5


def ulp16(y_bits):
    """Spacing of fp16 numbers at |y| (y given as fp16 bit patterns): 2^(e - 10) for
    2^e <= |y| < 2^(e + 1), and 2^-24 in the subnormal range."""
    a = np.abs(np.asarray(y_bits, np.uint16).view(np.float16).astype(np.float64))
    _, ex = np.frexp(a)                       # a = m * 2^ex, 0.5 <= m < 1
    e = np.where(a == 0, -14, np.maximum(ex.astype(np.int64) - 1, -14))
    return np.ldexp(1.0, e - 10)


def check(y_gpu_bits, y_ref_bits, acc_gpu, acc_ref, S):
    """Returns (every output passes, outputs beyond one ulp, outputs whose fp32 sum is
    off by more than REL * S).  Arrays of one shape; y as fp16 bit patterns."""
    gb = np.asarray(y_gpu_bits, np.uint16)
    rb = np.asarray(y_ref_bits, np.uint16)
    yg = gb.view(np.float16).astype(np.float64)
    yr = rb.view(np.float16).astype(np.float64)
    # equal bits agree (also where both overflowed to the same infinity, whose
    # difference is not a number)
    with np.errstate(invalid="ignore"):
        within_ulp = (gb == rb) | (np.abs(yg - yr) <= ulp16(rb))
    acc_ok = np.abs(np.asarray(acc_gpu, np.float64) - np.asarray(acc_ref, np.float64)) <= \
        REL * np.asarray(S, np.float64)
    ok = within_ulp | acc_ok
    return bool(np.all(ok)), int(np.sum(~within_ulp)), int(np.sum(~acc_ok))
