"""GPU parity at the edges of the documented size limits.

* K at its maximum (2^22 = 4,194,304, i.e. 32768 groups): every 32-bit buffer
  offset the kernels form is largest here (row x K for the activation rows a
  prefill tile covers, tile x 12K for the packed weights, group x M for the scale
  columns).  Two token rows through the decode kernel and each prefill tile, both
  precisions, checked against the oracle over the whole output.
* A very wide layer (N = 2^20 output columns, one group deep): a million 16-column
  decode work items and 8192 to 16384 prefill column tiles in one grid, checked on
  a sample of columns at the start, the middle and the end.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
G = 128
MAX_K = 1 << 22


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("abits", [6, 8])
def test_maximum_k(fq, abits):
    M, N, K = 2, 16, MAX_K
    nt = synth.default_threads()
    x = synth.activations(synth.derive_seed(41, "x", abits), M, K, nthreads=nt)
    w = synth.weights(synth.derive_seed(41, "w"), N, K, nthreads=nt)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qw_ref, sw_ref = oracle.quant_w6(w)
    y_ref = oracle.gemm(qa_ref, sa_ref, qw_ref, sw_ref).view(np.uint16)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    del w
    qa, sa = fq.quant_act(torch.from_numpy(x).to(DEV), abits)
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), sa_ref.view(np.uint32))
    for path in (fq.PATH_DECODE, fq.PATH_PREFILL_256X128, fq.PATH_PREFILL_128X128,
                 fq.PATH_PREFILL_128X64, fq.PATH_PREFILL_256X128_WS, fq.PATH_PREFILL_64X128):
        say(f"K = 2^22 abits={abits} path={path}")
        y = fq.gemm_w6ax(qa, sa, wp, sw, N, abits, path=path)
        assert np.array_equal(y.cpu().numpy().view(np.uint16), y_ref), f"path {path}"


@pytest.mark.parametrize("M", [1, 130])
def test_very_wide_layer(fq, M):
    N, K = 1 << 20, G
    nt = synth.default_threads()
    x = synth.activations(synth.derive_seed(42, "x", M), M, K, nthreads=nt)
    w = synth.weights(synth.derive_seed(42, "w"), N, K, nthreads=nt)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    qa, sa = fq.quant_act(torch.from_numpy(x).to(DEV), 6)
    tiles = np.array([0, 1, N // 32, N // 16 - 2, N // 16 - 1])
    cols = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tiles])
    qa_ref, sa_ref = oracle.quant_act(x, 6)
    qw_ref, sw_ref = oracle.quant_w6(np.ascontiguousarray(w[cols]))
    del w
    y_ref = oracle.gemm(qa_ref, sa_ref, qw_ref, sw_ref).view(np.uint16)
    for path in (fq.PATH_DECODE, fq.PATH_PREFILL):
        say(f"N = 2^20 M={M} path={path}")
        y = fq.gemm_w6ax(qa, sa, wp, sw, N, 6, path=path)
        got = y[:, torch.from_numpy(cols).to(DEV)].cpu().numpy().view(np.uint16)
        bad = np.argwhere(got != y_ref)
        assert bad.size == 0, f"path {path}: {len(bad)} sampled outputs differ"
