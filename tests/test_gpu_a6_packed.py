"""GPU parity of the 6-bit activation storage (FlexQ abstract: W6A6 holds the
activations at 6 bits) against the CPU oracle.

* flexq_quant_act_a6_packed: the packed codes equal the oracle's packing of its own
  A6 codes (oracle.pack_act_a6 of oracle.quant_act(x, 6)) word for word, and the
  scales equal its scales bit for bit, on random rows, edge values and quotients on
  rounding boundaries; nothing outside the two outputs is written.
* flexq_gemm_w6a6_packed: Y equals the oracle's Y on the unpacked codes bit for bit,
  and the byte-per-code streaming kernel's Y, on shapes that reach every kernel
  configuration the streaming GEMM picks (1 to 64 rows per pass, single and paired
  16-column tiles, chunks of 1 to 8 items, the 8- and 16-wave folds), ragged N, and
  M above one 64-row pass.
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


def check_quant(fq, x):
    qa_ref, sa_ref = oracle.quant_act(x, 6)
    qp_ref = oracle.pack_act_a6(qa_ref)
    qp, sa = fq.quant_act_a6_packed(to_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))
    got = qp.cpu().numpy().view(np.uint32)
    bad = np.argwhere(got != qp_ref)
    first = [(int(b[0]), int(b[1]) // 3) for b in bad[:4]]
    assert bad.size == 0, f"{len(bad)} words differ, first (row, unit) {first}"
    return qa_ref, sa_ref


@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (16, 8192), (64, 1152), (100, 2816),
                                 (5, 28672), (1, 16512)])
def test_quant_packed_bit_exact(fq, M, K):
    say(f"quant_act_a6_packed M={M} K={K}")
    check_quant(fq, synth.activations(synth.derive_seed(31, M, K), M, K))


def test_quant_packed_edge_values(fq):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((6, 3 * G)).astype(np.float16)
    x[0, :G] = 0
    x[1, :G] = np.float16(2.0 ** -24) * np.sign(rng.standard_normal(G)).astype(np.float16)
    x[2, :G] = np.float16(65504.0)
    x[2, 3] = np.float16(-65504.0)
    x[3, :G] = (np.arange(G) - 64).astype(np.float16) * np.float16(0.5)
    x[4, G:2 * G] = (rng.standard_normal(G) * 1e-7).astype(np.float16)
    qa_ref, _ = check_quant(fq, x)
    assert qa_ref.min() == -31 and qa_ref.max() == 31     # both ends of the A6 range


def test_quant_packed_quotients_on_rounding_boundaries(fq):
    rows = []
    for e in (-4, 0, 3):
        s = 2.0 ** e
        k = np.arange(-31, 31, dtype=np.float64) + 0.5
        ties = (k * s).astype(np.float16)
        for vals in (ties, np.nextafter(ties, np.float16(np.inf)),
                     np.nextafter(ties, np.float16(-np.inf))):
            row = np.zeros(G, dtype=np.float16)
            row[0] = np.float16(31 * s)
            row[1:1 + len(vals)] = vals
            rows.append(row)
    check_quant(fq, np.stack(rows))


def test_quant_packed_writes_stay_inside_the_outputs(fq):
    M, K = 7, 1280
    x = synth.activations(synth.derive_seed(32, M, K), M, K)
    qa_ref, sa_ref = oracle.quant_act(x, 6)
    pad = 64
    words = 3 * K // 16
    qbuf = torch.full((M * words + 2 * pad,), -1, dtype=torch.int32, device=DEV)
    sbuf = torch.full((M * (K // G) + 2 * pad,), -1, dtype=torch.int32, device=DEV)
    qp = qbuf[pad:pad + M * words].view(M, words)
    sa = sbuf[pad:pad + M * (K // G)].view(torch.float32).view(K // G, M)
    fq.quant_act_a6_packed(to_dev(x), q_a6p=qp, s_a=sa)
    torch.cuda.synchronize()
    for buf in (qbuf, sbuf):
        assert bool(torch.all(buf[:pad] == -1)) and bool(torch.all(buf[-pad:] == -1))
    assert np.array_equal(qp.cpu().numpy().view(np.uint32), oracle.pack_act_a6(qa_ref))
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))


# (M, N, K) on 256 compute units: narrow short layers (single 16-column tiles; up to
# 4 rows chunks of 1 or 2 items, from 5 rows chunks of 1, 2 or 4), more than 2 single
# tiles per CU (paired tiles, chunks of 2), deep K or wide N (paired tiles, 16 waves
# up to 4 rows, 8 waves from 5, chunks of 1, 2 or 8), 17-32 rows (paired tiles in
# chunks of 1, 2 or 8), 33-48 and 49-64 rows (chunks of 1 or 4), and two passes of
# 64 rows (chunks of 1 and 8)
GEMM_SHAPES = [(1, 256, 1024), (4, 400, 2048), (4, 4608, 1024), (5, 272, 1152),
               (16, 1024, 4096), (8, 4608, 1024), (16, 8704, 1024), (3, 8448, 1024),
               (2, 256, 16512), (9, 512, 16512), (16, 144, 17920), (12, 13312, 1024),
               (6, 33024, 256), (17, 496, 2048), (32, 2048, 1024), (30, 8704, 512),
               (24, 256, 16512), (20, 33024, 256), (40, 1040, 2048), (48, 272, 3072),
               (36, 16416, 256), (60, 2064, 1024), (64, 512, 1280), (130, 528, 1152),
               (100, 16416, 256)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_packed_bit_exact(fq, M, N, K):
    say(f"gemm_w6a6_packed M={M} N={N} K={K}")
    seed = synth.derive_seed(33, M, N, K)
    x = synth.activations(synth.derive_seed(seed, "x"), M, K)
    w = synth.weights(synth.derive_seed(seed, "w"), N, K)
    qa_ref, sa_ref = oracle.quant_act(x, 6)
    wp_ref, sw_ref = oracle.pack_w6(w)
    y_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N)
    qp = to_dev(oracle.pack_act_a6(qa_ref).view(np.int32))
    sa = to_dev(gm(sa_ref))
    wp = to_dev(wp_ref.view(np.int32))
    sw = to_dev(gm(sw_ref))
    y = fq.gemm_w6a6_packed(qp, sa, wp, sw, N)
    y_bytes = fq.gemm_w6ax(to_dev(qa_ref), sa, wp, sw, N, 6, path=fq.PATH_DECODE)
    torch.cuda.synchronize()
    got = y.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != y_ref.view(np.uint16))
    assert bad.size == 0, f"{len(bad)} of {got.size} differ, first {bad[:4].tolist()}"
    assert torch.equal(y.view(torch.int16), y_bytes.view(torch.int16))


def test_quant_then_gemm_packed_equals_the_byte_path(fq):
    """The two packed calls give the scales of quant_act(x, 6) and the Y of the
    streaming GEMM over its byte codes, here on full 8192-deep rows."""
    for M, N, K in [(16, 1024, 8192), (3, 1024, 8192)]:
        seed = synth.derive_seed(34, M, N, K)
        x = to_dev(synth.activations(synth.derive_seed(seed, "x"), M, K))
        wp, sw = fq.pack_w6(to_dev(synth.weights(synth.derive_seed(seed, "w"), N, K)))
        qp, sap = fq.quant_act_a6_packed(x)
        yp = fq.gemm_w6a6_packed(qp, sap, wp, sw, N)
        qa, sa = fq.quant_act(x, 6)
        yb = fq.gemm_w6ax(qa, sa, wp, sw, N, 6, path=fq.PATH_DECODE)
        torch.cuda.synchronize()
        assert torch.equal(sap.view(torch.int32), sa.view(torch.int32))
        assert torch.equal(yp.view(torch.int16), yb.view(torch.int16))


def test_gemm_packed_every_code(fq):
    """Codes the quantizer never produces still decode as the unit encoding says: a
    packed activation holding every code -32 .. 31, and a row of -32 throughout
    (against weights whose every group holds a code of magnitude 31, its maximum),
    gives the oracle's Y on those codes."""
    M, N, K = 5, 272, 1024
    rng = np.random.default_rng(35)
    qa = rng.integers(-32, 32, (M, K)).astype(np.int8)
    qa[0, :64] = np.arange(-32, 32)
    qa[1] = -32
    w = synth.weights(synth.derive_seed(35, "w"), N, K)
    wp_ref, sw_ref = oracle.pack_w6(w)
    sa_ref = (rng.random((M, K // G)) + 0.5).astype(np.float32) * np.float32(0.01)
    y_ref = oracle.gemm_packed(qa, sa_ref, wp_ref, sw_ref, N)
    y = fq.gemm_w6a6_packed(to_dev(oracle.pack_act_a6(qa).view(np.int32)), to_dev(gm(sa_ref)),
                            to_dev(wp_ref.view(np.int32)), to_dev(gm(sw_ref)), N)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), y_ref.view(np.uint16))
