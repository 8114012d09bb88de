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
# (128 x 64 tiles at these sizes) and by name with 256 x 128, 128 x 128 and 64 x 128
# tiles
CASES = [(1, 512, 1024, 6, 0), (16, 1040, 2048, 8, 0), (40, 208, 1024, 6, 0),
         (300, 400, 768, 8, 0), (1100, 144, 384, 6, 0), (300, 400, 768, 6, 3),
         (1100, 144, 384, 8, 4), (60, 400, 1152, 8, 7)]
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


def test_splitk_graph_replays_match_eager(fq):
    """The split-K GEMM (slice kernel + ordered reduce) captured in a HIP graph, as the
    benchmark captures it: every replay, between eager work that poisons Y, the
    accumulator and the workspace, gives the eager bits, and those are within the
    tolerance of the oracle."""
    import tolerance
    cases = [(64, 1024, 4096, 8, 0, 2), (130, 400, 1280, 6, 3, 3), (60, 400, 1152, 6, 4, 7)]
    bufs = []
    for i, (M, N, K, abits, splits, path) in enumerate(cases):
        path = path if path >= 3 else fq.PATH_PREFILL
        x = synth.activations(synth.derive_seed(23, "x", i), M, K)
        w = synth.weights(synth.derive_seed(23, "w", i), N, K)
        qa_ref, sa_ref = oracle.quant_act(x, abits)
        wp_ref, sw_ref = oracle.pack_w6(w)
        ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N, want_acc=True)
        dev = [torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
               for a in (qa_ref, sa_ref.T, wp_ref.view(np.int32), sw_ref.T)]
        ws = torch.empty(max(16, fq.splitk_workspace_bytes(M, N, K, splits)), dtype=torch.uint8,
                         device=DEV)
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
        bufs.append((M, N, K, abits, splits, path, dev, ws, y, acc, ref))

    def run():
        for (M, N, K, abits, splits, path, dev, ws, y, acc, _) in bufs:
            fq.gemm_w6ax_splitk(*dev, N, abits, splits=splits, path=path, y=y, acc=acc,
                                workspace=ws)

    run()
    torch.cuda.synchronize()
    eager = [(y.clone(), acc.clone()) for (*_, y, acc, _) in bufs]
    for (M, N, K, abits, splits, path, dev, ws, y, acc, ref), (ye, ae) in zip(bufs, eager):
        ok, _, n_acc = tolerance.check(ye.cpu().numpy().view(np.uint16), ref[0].view(np.uint16),
                                       ae.cpu().numpy(), ref[1], ref[2])
        assert ok and n_acc == 0, (M, N, K, splits, path)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for (*_, ws, y, acc, _) in bufs:
            y.fill_(float("nan"))
            acc.fill_(float("nan"))
            ws.fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((*_, y, acc, _), (ye, ae)) in enumerate(zip(bufs, eager)):
            assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), f"replay {rep} case {i}: y"
            assert torch.equal(acc.view(torch.int32), ae.view(torch.int32)), \
                f"replay {rep} case {i}: acc"


def test_a6_packed_graph_replays_match_eager(fq):
    """The packed A6 quantizer and the streaming GEMM over its output, captured in one
    HIP graph: every replay, between eager work that poisons the packed codes, the
    scales and Y, gives the eager bits, and those equal the oracle's."""
    cases = [(1, 512, 1024), (16, 1040, 2048), (64, 400, 1152)]
    bufs = []
    for i, (M, N, K) in enumerate(cases):
        x = synth.activations(synth.derive_seed(24, "x", i), M, K)
        w = synth.weights(synth.derive_seed(24, "w", i), N, K)
        qa_ref, sa_ref = oracle.quant_act(x, 6)
        wp_ref, sw_ref = oracle.pack_w6(w)
        ref = (oracle.pack_act_a6(qa_ref), sa_ref,
               oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N))
        wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
        qp = torch.empty((M, 3 * K // 16), dtype=torch.int32, device=DEV)
        sa = torch.empty((K // G, M), dtype=torch.float32, device=DEV)
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        bufs.append((N, torch.from_numpy(x).to(DEV), wp, sw, qp, sa, y, ref))

    def run():
        for (N, xd, wp, sw, qp, sa, y, _) in bufs:
            fq.quant_act_a6_packed(xd, q_a6p=qp, s_a=sa)
            fq.gemm_w6a6_packed(qp, sa, wp, sw, N, y=y)

    run()
    torch.cuda.synchronize()
    for (N, xd, wp, sw, qp, sa, y, (qp_ref, sa_ref, y_ref)) in bufs:
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), qp_ref)
        assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), sa_ref.view(np.uint32))
        assert np.array_equal(y.cpu().numpy().view(np.uint16), y_ref.view(np.uint16))
    eager = [(qp.clone(), sa.clone(), y.clone()) for (_, _, _, _, qp, sa, y, _) in bufs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for (_, _, _, _, qp, sa, y, _) in bufs:
            qp.fill_(-1)
            sa.fill_(float("nan"))
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((_, _, _, _, qp, sa, y, _), (qe, se, ye)) in enumerate(zip(bufs, eager)):
            assert torch.equal(qp, qe), f"replay {rep} case {i}: packed codes"
            assert torch.equal(sa.view(torch.int32), se.view(torch.int32)), \
                f"replay {rep} case {i}: scales"
            assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), f"replay {rep} case {i}: y"


def test_blocked_graph_replays_match_eager(fq):
    """The blocked-code quantizer and the streaming GEMM over its output in one HIP
    graph: every replay, between eager work that poisons codes, scales and Y, gives
    the eager bits, and those equal the oracle's."""
    cases = [(1, 512, 1024, 6), (17, 1040, 2048, 8), (64, 400, 1152, 6)]
    bufs = []
    for i, (M, N, K, abits) in enumerate(cases):
        x = synth.activations(synth.derive_seed(25, "x", i), M, K)
        w = synth.weights(synth.derive_seed(25, "w", i), N, K)
        qa_ref, sa_ref = oracle.quant_act(x, abits)
        wp_ref, sw_ref = oracle.pack_w6(w)
        ref = (oracle.block_act(qa_ref), sa_ref,
               oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N))
        wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
        qb = torch.empty(fq.blocked_act_bytes(M, K), dtype=torch.int8, device=DEV)
        sa = torch.empty((K // G, M), dtype=torch.float32, device=DEV)
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        bufs.append((N, abits, torch.from_numpy(x).to(DEV), wp, sw, qb, sa, y, ref))

    def run():
        for (N, abits, xd, wp, sw, qb, sa, y, _) in bufs:
            fq.quant_act_blocked(xd, abits, q_a_blk=qb, s_a=sa)
            fq.gemm_w6ax_blocked(qb, sa, wp, sw, N, abits, y=y)

    run()
    torch.cuda.synchronize()
    for (N, abits, xd, wp, sw, qb, sa, y, (qb_ref, sa_ref, y_ref)) in bufs:
        assert np.array_equal(qb.cpu().numpy(), qb_ref)
        assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), sa_ref.view(np.uint32))
        assert np.array_equal(y.cpu().numpy().view(np.uint16), y_ref.view(np.uint16))
    eager = [(qb.clone(), sa.clone(), y.clone()) for (*_, qb, sa, y, _) in bufs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for (*_, qb, sa, y, _) in bufs:
            qb.fill_(-1)
            sa.fill_(float("nan"))
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, ((*_, qb, sa, y, _), (qe, se, ye)) in enumerate(zip(bufs, eager)):
            assert torch.equal(qb, qe), f"replay {rep} case {i}: codes"
            assert torch.equal(sa.view(torch.int32), se.view(torch.int32)), \
                f"replay {rep} case {i}: scales"
            assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), f"replay {rep} case {i}: y"
