"""GPU parity of the split-K GEMM (flexq_gemm_w6ax_splitk) against the CPU oracle.

K is cut into S slices at group boundaries; each slice accumulates its groups from
+0 with the definition's t / fma steps and the fp32 slice sums are added in
ascending order.  So:

* S = 1 is the definition itself: Y and the fp32 accumulator bit for bit, on every
  tile (256 x 128, 128 x 128, 128 x 64, 64 x 128);
* S > 1 changes only the fp32 summation order: every output within one fp16 ulp or
  its fp32 sum within 1e-5 * sum |t * s_a| of the sequential accumulator (the
  tolerance module), and in these cases every fp32 sum within that bound;
* the result is the same bits on every call;
* nothing outside Y, the accumulator and the stated workspace is written, and Y is
  written everywhere.

Shapes are ragged in M and N (partial tiles in both directions), with K from one
group to 22 and S from 1 to one group per slice.
"""
import numpy as np
import pytest

import oracle
import synth
import tolerance

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
# (M, N, K)
SHAPES = [(64, 256, 1024), (100, 144, 1280), (257, 272, 2048), (1, 16, 128), (130, 64, 384),
          (37, 400, 2816)]
TILES = (3, 4, 5, 7)   # PATH_PREFILL_256X128, _128X128, _128X64, _64X128


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gm(a):
    return np.ascontiguousarray(np.asarray(a).T)


_cache = {}


def case(M, N, K, abits):
    """Oracle inputs and results (Y bits, fp32 accumulator, S) for one shape, and the
    same operands on the GPU."""
    key = (M, N, K, abits)
    if key not in _cache:
        seed = synth.derive_seed(synth.BASE_SEED, "splitk", M, N, K)
        x = synth.activations(synth.derive_seed(seed, "x"), M, K)
        w = synth.weights(synth.derive_seed(seed, "w"), N, K)
        qa, sa = oracle.quant_act(x, abits)
        wp, sw = oracle.pack_w6(w)
        y, acc, S = oracle.gemm_packed(qa, sa, wp, sw, N, want_acc=True)
        dev = [to_dev(qa), to_dev(gm(sa)), to_dev(wp.view(np.int32)), to_dev(gm(sw))]
        _cache.clear()
        _cache[key] = (dev, y.view(np.uint16), acc.astype(np.float32), S)
    return _cache[key]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("abits", (6, 8))
def test_one_slice_is_the_definition(fq, M, N, K, abits):
    dev, y_ref, acc_ref, _ = case(M, N, K, abits)
    for path in TILES:
        say(f"splitk S=1 M={M} N={N} K={K} abits={abits} tile path {path}")
        acc = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        y = fq.gemm_w6ax_splitk(*dev, N, abits, splits=1, path=path, acc=acc)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy().view(np.uint16), y_ref)
        assert np.array_equal(acc.cpu().numpy().view(np.uint32), acc_ref.view(np.uint32))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("abits", (6, 8))
def test_slices_within_tolerance(fq, M, N, K, abits):
    dev, y_ref, acc_ref, S_ref = case(M, N, K, abits)
    G = K // 128
    for path in TILES:
        for S in sorted({2, 3, 5, G}):
            if S < 2 or S > G:
                continue
            say(f"splitk S={S} M={M} N={N} K={K} abits={abits} tile path {path}")
            acc = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
            y = fq.gemm_w6ax_splitk(*dev, N, abits, splits=S, path=path, acc=acc)
            torch.cuda.synchronize()
            ok, n_ulp, n_acc = tolerance.check(y.cpu().numpy().view(np.uint16), y_ref,
                                               acc.cpu().numpy(), acc_ref, S_ref)
            assert ok and n_acc == 0, (n_ulp, n_acc)
            # Y is the fp16 rounding of the accumulator the call reports
            acc_h = acc.cpu().numpy().astype(np.float16).view(np.uint16)
            assert np.array_equal(y.cpu().numpy().view(np.uint16), acc_h)


def test_deterministic(fq):
    M, N, K = 257, 272, 2048
    dev, _, _, _ = case(M, N, K, 6)
    runs = []
    for _ in range(3):
        acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
        y = fq.gemm_w6ax_splitk(*dev, N, 6, splits=5, path=4, acc=acc)
        torch.cuda.synchronize()
        runs.append((y.cpu().numpy().view(np.uint16).copy(), acc.cpu().numpy().view(np.uint32).copy()))
    for y, a in runs[1:]:
        assert np.array_equal(y, runs[0][0]) and np.array_equal(a, runs[0][1])


def test_planned_split(fq):
    """splits = 0 and path PREFILL take the plan; on a mid-sized, narrow product the
    plan splits, and the result is within the tolerance."""
    M, N, K = 64, 1024, 4096
    S, tile = fq.splitk_plan(M, N, K)
    say(f"plan for M={M} N={N} K={K}: S={S} tile path {tile}")
    assert S > 1
    dev, y_ref, acc_ref, S_ref = case(M, N, K, 8)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y = fq.gemm_w6ax_splitk(*dev, N, 8, acc=acc)
    torch.cuda.synchronize()
    ok, _, n_acc = tolerance.check(y.cpu().numpy().view(np.uint16), y_ref, acc.cpu().numpy(),
                                   acc_ref, S_ref)
    assert ok and n_acc == 0
    # the same call with the plan's values spelled out gives the same bits
    y2 = fq.gemm_w6ax_splitk(*dev, N, 8, splits=S, path=tile)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_writes_stay_inside_the_outputs(fq):
    """Y, the accumulator and an exactly sized workspace sit inside larger buffers
    filled with a marker; after the call every marker byte outside them is intact
    and every Y and accumulator element was written."""
    M, N, K, S = 130, 144, 1280, 3
    dev, y_ref, acc_ref, S_ref = case(M, N, K, 6)
    pad = 256
    need = fq.splitk_workspace_bytes(M, N, K, S)
    assert need == S * M * N * 4
    wbuf = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV)
    ybuf = torch.full((M * N + 2 * pad,), -1, dtype=torch.int16, device=DEV)
    abuf = torch.full((M * N + 2 * pad,), -1, dtype=torch.int32, device=DEV)
    y = ybuf[pad:pad + M * N].view(torch.float16).view(M, N)
    acc = abuf[pad:pad + M * N].view(torch.float32).view(M, N)
    fq.gemm_w6ax_splitk(*dev, N, 6, splits=S, path=5, y=y, acc=acc,
                        workspace=wbuf[pad:pad + need])
    torch.cuda.synchronize()
    for buf, fill in ((wbuf, 0x5A), (ybuf, -1), (abuf, -1)):
        assert bool(torch.all(buf[:pad] == fill)) and bool(torch.all(buf[-pad:] == fill))
    assert not bool(torch.any(ybuf[pad:pad + M * N] == -1))
    assert not bool(torch.any(abuf[pad:pad + M * N] == -1))
    ok, _, n_acc = tolerance.check(y.cpu().numpy().view(np.uint16), y_ref, acc.cpu().numpy(),
                                   acc_ref, S_ref)
    assert ok and n_acc == 0


def test_without_accumulator_output(fq):
    M, N, K = 100, 144, 1280
    dev, _, _, _ = case(M, N, K, 8)
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y1 = fq.gemm_w6ax_splitk(*dev, N, 8, splits=4, path=3, acc=acc)
    y2 = fq.gemm_w6ax_splitk(*dev, N, 8, splits=4, path=3)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
