"""HIP graph capture of the layer path (activation quantization + GEMM).

Serving loops replay captured graphs instead of launching kernel by kernel; the
library's calls must capture and replay to the same bits.  A graph holding both
GEMM kernels (decode and prefill shapes, every prefill tile, A6 and A8) is replayed
several times, with unrelated eager work and synchronizations between replays;
every replay must reproduce the eager results bit for bit, and the eager results
are checked against the oracle on the prefill shapes.  The same graph holds two one-call
layers (flexq_linear_w6ax, q_a and s_a in a workspace), checked against the oracle.
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
# (M, N, K, abits, path): decode (1, 16, 40 rows); prefill by the automatic choice
# (128 x 64 tiles at these sizes) and by name with 256 x 128 and 128 x 128 tiles
CASES = [(1, 512, 1024, 6, 0), (16, 1040, 2048, 8, 0), (40, 208, 1024, 6, 0),
         (300, 400, 768, 8, 0), (1100, 144, 384, 6, 0), (300, 400, 768, 6, 3),
         (1100, 144, 384, 8, 4)]
LINEAR_CASES = [(2, 400, 1024, 8), (8, 208, 768, 6)]


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def test_graph_replays_match_eager(fq):
    bufs = []
    for i, (M, N, K, abits, path) in enumerate(CASES):
        x = synth.activations(synth.derive_seed(21, "x", i), M, K)
        w = synth.weights(synth.derive_seed(21, "w", i), N, K)
        wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
        xd = torch.from_numpy(x).to(DEV)
        qa = torch.empty((M, K), dtype=torch.int8, device=DEV)
        sa = torch.empty((K // G, M), dtype=torch.float32, device=DEV)
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        bufs.append((M, N, K, abits, path, x, w, xd, wp, sw, qa, sa, y))
    lin = []
    for i, (M, N, K, abits) in enumerate(LINEAR_CASES):
        x = synth.activations(synth.derive_seed(22, "x", i), M, K)
        w = synth.weights(synth.derive_seed(22, "w", i), N, K)
        wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
        ws = torch.empty(fq.linear_w6ax_workspace_bytes(M, K), dtype=torch.uint8, device=DEV)
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        lin.append((M, N, K, abits, x, w, torch.from_numpy(x).to(DEV), wp, sw, ws, y))

    def run():
        for (M, N, K, abits, path, x, w, xd, wp, sw, qa, sa, y) in bufs:
            fq.quant_act(xd, abits, q_a=qa, s_a=sa)
            fq.gemm_w6ax(qa, sa, wp, sw, N, abits, y=y, path=path)
        for (M, N, K, abits, x, w, xd, wp, sw, ws, y) in lin:
            fq.linear_w6ax(xd, wp, sw, N, abits, y=y, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [(qa.clone(), sa.clone(), y.clone()) for (*_, qa, sa, y) in bufs]
    lin_ref = [y.clone() for (*_, y) in lin]
    for (M, N, K, abits, x, w, *_), yr in zip(lin, lin_ref):
        qa_ref, sa_ref = oracle.quant_act(x, abits)
        wp_ref, sw_ref = oracle.pack_w6(w)
        y_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N)
        assert np.array_equal(yr.cpu().numpy().view(np.uint16), y_ref.view(np.uint16))

    # the eager results themselves, against the oracle, on the prefill cases
    for i in (3, 5, 6):
        M, N, K, abits, path, x, w = bufs[i][:7]
        qa_ref, sa_ref = oracle.quant_act(x, abits)
        wp_ref, sw_ref = oracle.pack_w6(w)
        y_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N)
        assert np.array_equal(ref[i][2].cpu().numpy().view(np.uint16), y_ref.view(np.uint16))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    scratch = torch.empty((64, 4096), dtype=torch.float16, device=DEV)
    for rep in range(4):
        for (*_, qa, sa, y) in bufs:   # poison the outputs eagerly between replays
            qa.fill_(-1)
            sa.fill_(float("nan"))
            y.fill_(float("nan"))
        for (*_, ws, y) in lin:
            y.fill_(float("nan"))
            ws.fill_(0xAB)
        scratch.normal_()              # unrelated eager work on the same stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((*_, qa, sa, y), (qr, sr, yr)) in enumerate(zip(bufs, ref)):
            assert torch.equal(qa, qr), f"replay {rep} case {CASES[i]}: q_a"
            assert torch.equal(sa.view(torch.int32), sr.view(torch.int32)), \
                f"replay {rep} case {CASES[i]}: s_a"
            assert torch.equal(y.view(torch.int16), yr.view(torch.int16)), \
                f"replay {rep} case {CASES[i]}: y"
        for i, ((*_, y), yr) in enumerate(zip(lin, lin_ref)):
            assert torch.equal(y.view(torch.int16), yr.view(torch.int16)), \
                f"replay {rep} linear case {LINEAR_CASES[i]}"
