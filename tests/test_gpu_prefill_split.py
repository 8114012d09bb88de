"""GPU parity of the prefill tail split.

Shapes whose 256 x 128 grid ends in a partly filled round of one tile per compute
unit run (PATH_PREFILL) as a 256 x 128 launch over the leading columns and a
128 x 64 launch over the rest, both writing into one Y.  The cases cover a split at
8192 of 10240 columns, ragged M and a ragged last tail tile (1000 x 10192), three
row blocks (520 rows), 32 row blocks and a one-block main launch (8192 x 1280, a
tensor-parallel qkv shard), and a tail of 1.5 tiles per compute unit
(1024 x 27648).  Each case checks that the split happens on this device (the
shapes are chosen for 256 compute units), then compares Y, written over a NaN
fill, with the oracle and with the single 256 x 128 launch bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
# (M, N, K, abits)
CASES = [(1024, 10240, 256, 6), (1000, 10192, 128, 8), (520, 33280, 128, 6),
         (8192, 1280, 128, 8), (1024, 27648, 128, 6)]


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


@pytest.mark.parametrize("M,N,K,abits", CASES)
def test_split_bit_exact(fq, M, N, K, abits):
    main = fq.prefill_main_cols(M, N, K)
    print(f"split M={M} N={N} K={K} abits={abits}: main launch {main} columns", flush=True)
    if main == N:
        pytest.skip("no tail split for this shape on this device's compute-unit count")
    assert 0 < main < N and main % 128 == 0
    i = CASES.index((M, N, K, abits))
    x = synth.activations(synth.derive_seed(71, "x", i), M, K)
    w = synth.weights(synth.derive_seed(71, "w", i), N, K)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    wp_ref, sw_ref = oracle.pack_w6(w)
    y_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N).view(np.uint16)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    qa, sa = fq.quant_act(torch.from_numpy(x).to(DEV), abits)
    ys = {}
    for path in (fq.PATH_PREFILL, fq.PATH_PREFILL_256X128):
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        fq.gemm_w6ax(qa, sa, wp, sw, N, abits, y=y, path=path)
        ys[path] = y.cpu().numpy().view(np.uint16)
    for path, got in ys.items():
        bad = np.argwhere(got != y_ref)
        assert bad.size == 0, f"path {path}: {len(bad)} mismatches, first at {bad[:4].tolist()}"
