"""GPU parity on seeded random shapes: every kernel and prefill tile on shapes drawn
to land on and around their boundaries.

Each case draws M in 1..320 (decode passes of 16/32/48/64 rows, prefill row tiles of
128 and 256, ragged tails), N a multiple of 16 in 16..2048 (odd and even tile
counts for single and paired decode tiles and for 64- and 128-wide prefill tiles),
K a multiple of 128 in 128..3072 (group counts below, at and past the 16 a decode
workgroup folds per round and the 6 a prefill loop unrolls), the activation
precision and the path (automatic, decode, automatic prefill tile, one named tile,
the warp-specialized kernel or the 64 x 128 tile).  Y and the activation codes and
scales must equal the oracle's bit for bit; every case also runs the blocked-code pair
(flexq_quant_act_blocked, flexq_gemm_w6ax_blocked) and A6 cases the packed pair
(flexq_quant_act_a6_packed, flexq_gemm_w6a6_packed) against the oracle's layouts and Y.
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
N_CASES = 48


def draw_cases():
    rng = np.random.default_rng(synth.derive_seed(51, "shapes") & 0xFFFFFFFF)
    cases = []
    for i in range(N_CASES):
        M = int(rng.choice([1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 127,
                            128, 129, 255, 256, 257, 320]))
        N = 16 * int(rng.integers(1, 129))
        K = G * int(rng.integers(1, 25))
        abits = int(rng.choice([6, 8]))
        path = int(rng.integers(0, 8))
        cases.append((i, M, N, K, abits, path))
    return cases


CASES = draw_cases()


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


@pytest.mark.parametrize("i,M,N,K,abits,path", CASES,
                         ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}-a{c[4]}-p{c[5]}" for c in CASES])
def test_random_shape_bit_exact(fq, i, M, N, K, abits, path):
    print(f"case {i}: M={M} N={N} K={K} abits={abits} path={path}", flush=True)
    x = synth.activations(synth.derive_seed(51, "x", i), M, K)
    w = synth.weights(synth.derive_seed(51, "w", i), N, K)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qw_ref, sw_ref = oracle.quant_w6(w)
    y_ref = oracle.gemm(qa_ref, sa_ref, qw_ref, sw_ref).view(np.uint16)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    xd = torch.from_numpy(x).to(DEV)
    qa, sa = fq.quant_act(xd, abits)
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), sa_ref.view(np.uint32))
    y = fq.gemm_w6ax(qa, sa, wp, sw, N, abits, path=path)
    got = y.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != y_ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    # codes in 16-row blocks: the oracle's blocking and the same Y
    qb, sab = fq.quant_act_blocked(xd, abits)
    yb = fq.gemm_w6ax_blocked(qb, sab, wp, sw, N, abits)
    assert np.array_equal(qb.cpu().numpy(), oracle.block_act(qa_ref))
    assert torch.equal(sab.view(torch.int32), sa.view(torch.int32))
    assert np.array_equal(yb.cpu().numpy().view(np.uint16), y_ref)
    if abits == 6:  # 6-bit activation storage: the oracle's packing and the same Y
        qp, sap = fq.quant_act_a6_packed(xd)
        yp = fq.gemm_w6a6_packed(qp, sap, wp, sw, N)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), oracle.pack_act_a6(qa_ref))
        assert torch.equal(sap.view(torch.int32), sa.view(torch.int32))
        assert np.array_equal(yp.cpu().numpy().view(np.uint16), y_ref)
