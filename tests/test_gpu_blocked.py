"""GPU parity of the blocked activation codes (16-row blocks in the order the
weight-streaming kernel feeds its MFMAs) against the CPU oracle.

* flexq_quant_act_blocked: the blocked codes equal the oracle's blocking of its own
  codes (oracle.block_act of oracle.quant_act) byte for byte, pad rows zero, and the
  scales equal its scales bit for bit, for A6 and A8, ragged M, edge values; nothing
  outside the two outputs is written.
* flexq_gemm_w6ax_blocked: Y equals the oracle's Y bit for bit, and the row-major
  streaming kernel's Y, on shapes that reach every configuration of the streaming
  kernel (1 to 64 rows per pass, single and paired tiles, chunks of 1 to 8 items, both
  folds) and M above one 64-row pass; pad rows holding garbage change nothing.
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


@pytest.mark.parametrize("M,K,abits", [(1, 128, 6), (5, 4096, 8), (16, 8192, 6), (17, 1152, 8),
                                       (64, 2816, 6), (100, 1280, 8), (3, 28672, 6)])
def test_quant_blocked_bit_exact(fq, M, K, abits):
    say(f"quant_act_blocked M={M} K={K} abits={abits}")
    x = synth.activations(synth.derive_seed(41, M, K), M, K)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    qb, sa = fq.quant_act_blocked(to_dev(x), abits)
    torch.cuda.synchronize()
    assert qb.numel() == fq.blocked_act_bytes(M, K) == (M + 15) // 16 * 16 * K
    got = qb.cpu().numpy()
    ref = oracle.block_act(qa_ref)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))


def test_quant_blocked_edge_values_and_guard_bands(fq):
    rng = np.random.default_rng(8)
    M, K = 6, 3 * G
    x = rng.standard_normal((M, K)).astype(np.float16)
    x[0, :G] = 0
    x[1, :G] = np.float16(2.0 ** -24)
    x[2, :G] = np.float16(65504.0)
    x[2, 3] = np.float16(-65504.0)
    x[3, :G] = (np.arange(G) - 64).astype(np.float16) * np.float16(0.5)
    for abits in (6, 8):
        qa_ref, sa_ref = oracle.quant_act(x, abits)
        pad = 64
        n = fq.blocked_act_bytes(M, K)
        qbuf = torch.full((n + 2 * pad,), 0x5A, dtype=torch.int8, device=DEV)
        sbuf = torch.full((M * (K // G) + 2 * pad,), -1, dtype=torch.int32, device=DEV)
        qb = qbuf[pad:pad + n]
        sa = sbuf[pad:pad + M * (K // G)].view(torch.float32).view(K // G, M)
        fq.quant_act_blocked(to_dev(x), abits, q_a_blk=qb, s_a=sa)
        torch.cuda.synchronize()
        assert bool(torch.all(qbuf[:pad] == 0x5A)) and bool(torch.all(qbuf[-pad:] == 0x5A))
        assert bool(torch.all(sbuf[:pad] == -1)) and bool(torch.all(sbuf[-pad:] == -1))
        assert np.array_equal(qb.cpu().numpy(), oracle.block_act(qa_ref))   # pad rows zero
        assert np.array_equal(sa.cpu().numpy().view(np.uint32), gm(sa_ref).view(np.uint32))


# the streaming kernel's configurations on 256 compute units, as in the packed-code test
GEMM_SHAPES = [(1, 256, 1024), (4, 400, 2048), (4, 4608, 1024), (5, 272, 1152),
               (16, 1024, 4096), (8, 4608, 1024), (16, 8704, 1024), (3, 8448, 1024),
               (2, 256, 16512), (9, 512, 16512), (16, 144, 17920), (12, 13312, 1024),
               (6, 33024, 256), (17, 496, 2048), (32, 2048, 1024), (30, 8704, 512),
               (24, 256, 16512), (20, 33024, 256), (40, 1040, 2048), (48, 272, 3072),
               (36, 16416, 256), (60, 2064, 1024), (64, 512, 1280), (130, 528, 1152),
               (100, 16416, 256)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_blocked_bit_exact(fq, M, N, K):
    abits = 6 if (M + N) % 2 else 8
    say(f"gemm_w6ax_blocked M={M} N={N} K={K} abits={abits}")
    seed = synth.derive_seed(43, M, N, K)
    x = synth.activations(synth.derive_seed(seed, "x"), M, K)
    w = synth.weights(synth.derive_seed(seed, "w"), N, K)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    wp_ref, sw_ref = oracle.pack_w6(w)
    y_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N)
    blk = oracle.block_act(qa_ref)
    Mp = (M + 15) // 16 * 16
    if Mp > M:   # pad rows with garbage: they only meet outputs that are never written
        blk.reshape(Mp // 16, K // G, 2, 16, 64)[-1, :, :, 16 - (Mp - M):, :] = 77
    sa = to_dev(gm(sa_ref))
    wp = to_dev(wp_ref.view(np.int32))
    sw = to_dev(gm(sw_ref))
    y = fq.gemm_w6ax_blocked(to_dev(blk), sa, wp, sw, N, abits)
    y_rm = fq.gemm_w6ax(to_dev(qa_ref), sa, wp, sw, N, abits, path=fq.PATH_DECODE)
    torch.cuda.synchronize()
    got = y.cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != y_ref.view(np.uint16))
    assert bad.size == 0, f"{len(bad)} of {got.size} differ, first {bad[:4].tolist()}"
    assert torch.equal(y.view(torch.int16), y_rm.view(torch.int16))


def test_quant_then_gemm_blocked_equals_the_row_major_pair(fq):
    for M, N, K, abits in [(16, 1024, 8192, 6), (3, 1024, 8192, 8), (64, 512, 28672, 8)]:
        seed = synth.derive_seed(44, M, N, K)
        x = to_dev(synth.activations(synth.derive_seed(seed, "x"), M, K))
        wp, sw = fq.pack_w6(to_dev(synth.weights(synth.derive_seed(seed, "w"), N, K)))
        qb, sab = fq.quant_act_blocked(x, abits)
        yb = fq.gemm_w6ax_blocked(qb, sab, wp, sw, N, abits)
        qa, sa = fq.quant_act(x, abits)
        yr = fq.gemm_w6ax(qa, sa, wp, sw, N, abits, path=fq.PATH_DECODE)
        torch.cuda.synchronize()
        assert torch.equal(sab.view(torch.int32), sa.view(torch.int32))
        assert torch.equal(yb.view(torch.int16), yr.view(torch.int16))
