"""GPU parity: every HIP entry point against the CPU oracle on the same seeded inputs.

Bit-exact everywhere: packed weights, weight scales, activation codes and scales,
int32 group dots, and Y (both GEMM kernels keep the sequential ascending-group
fp32 order of the definition, so Y matches to the last bit).
"""
import functools
import os

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

G = 128
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def u16(t):
    return t.cpu().numpy().view(np.uint16)


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def gm(a):
    """Oracle scales [rows][groups] -> the library's group-major [groups][rows]."""
    return np.ascontiguousarray(np.asarray(a).T)


def inputs(seed, M, N, K):
    x = synth.activations(synth.derive_seed(seed, "x", M, N, K), M, K)
    w = synth.weights(synth.derive_seed(seed, "w", M, N, K), N, K)
    return x, w


# ---------------------------------------------------------------------------
# pack_w6
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(16, 128), (256, 512), (48, 1152), (4096, 4096),
                                 (5120, 13824), (1024, 28672)])
def test_pack_w6_bit_exact(fq, N, K):
    say(f"pack_w6 N={N} K={K}")
    w = synth.weights(synth.derive_seed(1, N, K), N, K)
    wp_ref, sw_ref = oracle.pack_w6(w)
    wp, sw = fq.pack_w6(to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(u16(sw), gm(sw_ref).view(np.uint16))
    assert np.array_equal(u32(wp), wp_ref)


def test_pack_w6_edge_values(fq):
    """Zero groups, a group whose scale underflows in fp16, fp16 subnormals, the
    largest fp16 values, exact ties and sign flips."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((32, 4 * G)) * 0.02).astype(np.float16)
    w[0, :G] = 0                                   # zero group
    w[1, :G] = 0
    w[1, 5] = np.float16(2.0 ** -24)               # scale rounds to 0 in fp16
    w[2, :G] = (rng.standard_normal(G) * 1e-6).astype(np.float16)   # subnormal scale
    w[3, :G] = np.float16(65504.0) * np.sign(rng.standard_normal(G)).astype(np.float16)
    w[4, :G] = (np.arange(G) - 64).astype(np.float16) / np.float16(2)  # many ties
    w[5, G:2 * G] = -w[4, :G]
    wp_ref, sw_ref = oracle.pack_w6(w)
    wp, sw = fq.pack_w6(to_dev(w))
    assert np.array_equal(u16(sw), gm(sw_ref).view(np.uint16))
    assert np.array_equal(u32(wp), wp_ref)


# ---------------------------------------------------------------------------
# quant_act
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,abits", [(16, 512, 6), (1, 8192, 6), (1, 8192, 8), (77, 1280, 6),
                                       (64, 13824, 8), (2048, 8192, 6), (512, 28672, 8)])
def test_quant_act_bit_exact(fq, M, K, abits):
    say(f"quant_act M={M} K={K} abits={abits}")
    x = synth.activations(synth.derive_seed(2, M, K), M, K)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qa, sa = fq.quant_act(to_dev(x), abits)
    torch.cuda.synchronize()
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))
    assert np.array_equal(qa.cpu().numpy(), qa_ref)


@pytest.mark.parametrize("abits", [6, 8])
def test_quant_act_edge_values(fq, abits):
    rng = np.random.default_rng(abits)
    x = rng.standard_normal((6, 3 * G)).astype(np.float16)
    x[0, :G] = 0
    x[1, :G] = np.float16(2.0 ** -24) * np.sign(rng.standard_normal(G)).astype(np.float16)
    x[2, :G] = np.float16(65504.0)
    x[2, 3] = np.float16(-65504.0)
    x[3, :G] = (np.arange(G) - 64).astype(np.float16) * np.float16(0.5)
    x[4, G:2 * G] = (rng.standard_normal(G) * 1e-7).astype(np.float16)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qa, sa = fq.quant_act(to_dev(x), abits)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))
    assert np.array_equal(qa.cpu().numpy(), qa_ref)


@pytest.mark.parametrize("abits", [6, 8])
def test_quant_act_quotients_on_rounding_boundaries(fq, abits):
    """Groups whose quotients v / s are exactly k + 1/2 (ties to even) or one fp16
    step either side of it, where a quotient formed from the reciprocal of the
    scale lands next to the boundary and the kernel must take the exact one."""
    qmax = 31 if abits == 6 else 127
    rows = []
    for e in (-4, 0, 3):
        s = 2.0 ** e                        # s = amax / qmax exactly
        k = np.arange(-qmax, qmax, dtype=np.float64) + 0.5
        ties = (k * s).astype(np.float16)
        up = np.nextafter(ties, np.float16(np.inf))
        down = np.nextafter(ties, np.float16(-np.inf))
        for vals in (ties, up, down):
            row = np.zeros(2 * G, dtype=np.float16)
            row[0] = np.float16(qmax * s)     # the group maximum
            n = min(len(vals), G - 1)
            row[1:1 + n] = vals[:n]
            row[G] = np.float16(qmax * s)
            row[G + 1:G + 1 + len(vals) - n] = vals[n:]
            rows.append(row)
    x = np.stack(rows)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qa, sa = fq.quant_act(to_dev(x), abits)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))
    assert np.array_equal(qa.cpu().numpy(), qa_ref)


# ---------------------------------------------------------------------------
# group dots (unpack + MFMA lane mapping)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,abits", [(16, 256, 512, 6), (16, 256, 512, 8), (37, 80, 1024, 8),
                                         (1, 16, 128, 6), (64, 48, 2048, 6)])
def test_group_dots_bit_exact(fq, M, N, K, abits):
    say(f"group_dots M={M} N={N} K={K} abits={abits}")
    x, w = inputs(3, M, N, K)
    qa, _ = oracle.quant_act(x, abits)
    qw, _ = oracle.quant_w6(w)
    wp = oracle.pack_codes(qw)
    d_ref = oracle.group_dots(qa, qw)
    d = fq.gemm_w6ax_group_dots(to_dev(qa), to_dev(wp.view(np.int32)), N)
    assert np.array_equal(d.cpu().numpy(), d_ref)


def test_group_dots_extreme_codes(fq):
    """Every code of the format, including -32, against the integer matmul."""
    rng = np.random.default_rng(11)
    M, N, K = 16, 32, 4 * G
    qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-32, 32, (N, K)).astype(np.int8)
    qa[0] = 127
    qw[0] = -32
    qa[1] = -127
    qw[1] = 31
    wp = oracle.pack_codes(qw)
    d = fq.gemm_w6ax_group_dots(to_dev(qa), to_dev(wp.view(np.int32)), N)
    ref = np.stack([qa[:, g * G:(g + 1) * G].astype(np.int64) @
                    qw[:, g * G:(g + 1) * G].astype(np.int64).T for g in range(4)], axis=2)
    assert np.array_equal(d.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# GEMM: both kernels, many shapes, bit-exact Y
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=4)
def oracle_gemm_case(M, N, K, abits, seed):
    x, w = inputs(seed, M, N, K)
    qa, sa = oracle.quant_act(x, abits)
    wp, sw = oracle.pack_w6(w)
    return qa, sa, wp, sw, oracle.gemm_packed(qa, sa, wp, sw, N)


def run_gemm_case(fq, M, N, K, abits, path, seed=4):
    qa, sa, wp, sw, y_ref = oracle_gemm_case(M, N, K, abits, seed)
    y = fq.gemm_w6ax(to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw)), N,
                     abits, path=path)
    got = u16(y)
    bad = np.argwhere(got != y_ref.view(np.uint16))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


# (the wide shapes make the decode kernel pair adjacent column tiles, with a
# half-empty last pair, and give each workgroup 2 to 5 work items, so the items of a
# workgroup share their activation fragments in chunks of 2, 4 and 8; with 300 rows
# the chunks are also cut where a workgroup's items cross into the next 64-row pass.
# Every shape also runs each prefill tile (256 x 128, 128 x 128, 128 x 64) by name,
# on ragged row and column counts; the last two take the 256-row tile by the
# automatic choice.)
SHAPES = [(16, 256, 512), (1, 16, 128), (5, 48, 1152), (17, 272, 640), (33, 160, 384),
          (64, 128, 2048), (65, 144, 512), (128, 256, 1024), (130, 400, 768), (257, 96, 256),
          (300, 528, 1280), (1024, 256, 512), (1100, 400, 384), (2048, 128, 1024),
          (7, 16368, 256), (20, 16368, 384), (3, 20480, 384), (9, 40992, 256),
          (300, 16368, 256), (256, 16384, 256), (1024, 8192, 256)]


@pytest.mark.parametrize("path", [1, 2, 3, 4, 5, 6, 7],
                         ids=["decode", "prefill", "tile256x128", "tile128x128", "tile128x64",
                              "tile256x128ws", "tile64x128"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_bit_exact_every_path(fq, M, N, K, path):
    say(f"gemm M={M} N={N} K={K} path={path}")
    run_gemm_case(fq, M, N, K, 6 if (M + N) % 2 else 8, path)


@pytest.mark.parametrize("M", [1, 16, 64, 200])
def test_gemm_auto_path(fq, M):
    run_gemm_case(fq, M, 96, 1024, 8, 0)


def test_gemm_zero_rows_and_zero_groups(fq):
    """An all-zero activation group (s_a = 0), an all-zero weight group (s_w = 0)."""
    M, N, K = 20, 64, 3 * G
    x, w = inputs(9, M, N, K)
    x[3] = 0
    x[5, G:2 * G] = 0
    w[7] = 0
    w[9, :G] = 0
    for path in (1, 3, 4, 5, 6, 7):   # decode, then each prefill tile
        qa, sa = oracle.quant_act(x, 6)
        wp, sw = oracle.pack_w6(w)
        y_ref = oracle.gemm_packed(qa, sa, wp, sw, N)
        y = fq.gemm_w6ax(to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw)), N,
                         6, path=path)
        assert np.array_equal(u16(y), y_ref.view(np.uint16))


def test_gemm_deterministic_and_in_bounds(fq):
    """Two runs give identical bits; poisoned output is fully overwritten; guard
    bands after the output stay untouched."""
    M, N, K = 40, 208, 1024
    x, w = inputs(10, M, N, K)
    qa, sa = oracle.quant_act(x, 8)
    wp, sw = oracle.pack_w6(w)
    args = (to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw)))
    for path in (1, 3, 4, 5, 6, 7):   # decode, then each prefill tile
        buf = torch.full((M * N + 4096,), -1, dtype=torch.int16, device=DEV)
        y = buf[:M * N].view(torch.float16).view(M, N)
        fq.gemm_w6ax(*args, N, 8, y=y, path=path)
        first = u16(y).copy()
        fq.gemm_w6ax(*args, N, 8, y=y, path=path)
        assert np.array_equal(first, u16(y))
        assert not np.any(first == 0xFFFF)
        assert torch.all(buf[M * N:] == -1)


@pytest.mark.parametrize("M,N,K", [(40, 208, 1024), (1100, 144, 384)])
def test_gemm_output_not_16_byte_aligned(fq, M, N, K):
    """An output that is only 4-byte aligned (the documented minimum) takes the
    kernels' element-wise store path; the results and the guard bands around the
    output are the same as for an aligned one."""
    x, w = inputs(11, M, N, K)
    qa, sa = oracle.quant_act(x, 6)
    wp, sw = oracle.pack_w6(w)
    y_ref = oracle.gemm_packed(qa, sa, wp, sw, N).view(np.uint16)
    args = (to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw)))
    for path in (1, 3, 4, 5, 6, 7):   # decode, then each prefill tile
        buf = torch.full((M * N + 4096,), -1, dtype=torch.int16, device=DEV)
        y = buf[2:2 + M * N].view(torch.float16).view(M, N)   # 4 bytes past a 16-byte boundary
        assert y.data_ptr() % 16 == 4
        fq.gemm_w6ax(*args, N, 6, y=y, path=path)
        assert np.array_equal(u16(y), y_ref)
        assert torch.all(buf[:2] == -1) and torch.all(buf[2 + M * N:] == -1)


def test_end_to_end_layer(fq):
    """fp16 X and W through the three entry points equal the oracle's chain."""
    M, N, K = 24, 320, 1536
    x, w = inputs(12, M, N, K)
    for abits in (6, 8):
        layer = fq.W6AxLinear(to_dev(w), abits=abits)
        y = layer(to_dev(x))
        qa, sa = oracle.quant_act(x, abits)
        wp, sw = oracle.pack_w6(w)
        assert np.array_equal(u16(y), oracle.gemm_packed(qa, sa, wp, sw, N).view(np.uint16))


def test_stream_argument_is_honoured(fq):
    M, N, K = 16, 256, 512
    x, w = inputs(13, M, N, K)
    qa, sa = oracle.quant_act(x, 6)
    wp, sw = oracle.pack_w6(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d_qa, d_sa, d_wp, d_sw = (to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)),
                                  to_dev(gm(sw)))
        y = fq.gemm_w6ax(d_qa, d_sa, d_wp, d_sw, N, 6)
    s.synchronize()
    assert np.array_equal(u16(y), oracle.gemm_packed(qa, sa, wp, sw, N).view(np.uint16))


def test_stale_hip_error_does_not_fail_the_next_call(fq):
    """An error an earlier HIP call left in the thread's last-error slot is not
    reported as a failed launch: each call returns the status of its own launches
    (flexq.h, FLEXQ_ERROR_LAUNCH).  Covers the two-launch prefill tail split too."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")    # the HIP runtime torch and libflexq share
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    dev = torch.cuda.current_device()
    for M, N, K, path in [(5, 256, 512, fq.PATH_DECODE), (130, 256, 512, fq.PATH_PREFILL),
                          (1024, 10240, 256, fq.PATH_AUTO)]:
        x, w = inputs(14, M, N, K)
        qa, sa = oracle.quant_act(x, 8)
        wp, sw = oracle.pack_w6(w)
        args = (to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw)))
        torch.cuda.synchronize()
        assert hip.hipSetDevice(1 << 20) != 0      # an invalid device: a sticky error
        assert torch.cuda.current_device() == dev
        y = fq.gemm_w6ax(*args, N, 8, path=path)   # raises FlexqError on a non-zero status
        assert np.array_equal(u16(y), oracle.gemm_packed(qa, sa, wp, sw, N).view(np.uint16))
    assert fq.prefill_main_cols(1024, 10240, 256) < 10240   # the AUTO case ran the split
    hip.hipGetLastError()                         # leave the thread's error slot clear
