"""GPU parity under concurrent host threads: the C ABI called from several threads at
once, each thread enqueueing on a stream of its own (default priority).

Four threads start together and each runs one layer 16 times, rotating through the
one-call path (flexq_linear_w6ax, binding-allocated workspace), the two-call path
(flexq_quant_act, then flexq_gemm_w6ax), the split-K GEMM with one slice (its
own workspace), the blocked-code pair (flexq_quant_act_blocked, then
flexq_gemm_w6ax_blocked) and, for A6, the packed pair (flexq_quant_act_a6_packed, then
flexq_gemm_w6a6_packed), and querying the automatic path, the prefill tile and the split-K
plan before every call, so the per-device compute-unit cache is first filled while
the other threads use it.  The layers cover the decode kernel (1, 16
and 40 rows) and the prefill kernel (300 rows), A6 and A8.  Every output must equal
the oracle's bit for bit.
"""
import threading

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
# (M, N, K, abits)
CASES = [(1, 208, 1024, 6), (16, 1040, 2048, 8), (40, 144, 1152, 6), (300, 272, 768, 8)]
ITERS = 16


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def test_concurrent_threads_bit_exact(fq):
    prepared = []
    for i, (M, N, K, abits) in enumerate(CASES):
        x = synth.activations(synth.derive_seed(61, "x", i), M, K)
        w = synth.weights(synth.derive_seed(61, "w", i), N, K)
        qa, sa = oracle.quant_act(x, abits)
        wp, sw = oracle.pack_w6(w)
        y_ref = oracle.gemm_packed(qa, sa, wp, sw, N).view(np.uint16)
        wp_d, sw_d = fq.pack_w6(torch.from_numpy(w).to(DEV))
        prepared.append((M, N, K, abits, torch.from_numpy(x).to(DEV), wp_d, sw_d, y_ref))
    torch.cuda.synchronize()
    print(f"{len(CASES)} threads x {ITERS} calls", flush=True)

    results = [None] * len(CASES)
    errors = []
    start = threading.Barrier(len(CASES))

    def worker(i):
        try:
            M, N, K, abits, x, wp, sw, _ = prepared[i]
            stream = torch.cuda.Stream(device=DEV)
            outs = []
            start.wait(timeout=60)
            with torch.cuda.stream(stream):
                for it in range(ITERS):
                    fq.auto_path(M, N, K)
                    fq.prefill_tile(M, N, K)
                    fq.splitk_plan(M, N, K)
                    if it % 8 == 5:  # codes in 16-row blocks and the streaming GEMM
                        qb, sa = fq.quant_act_blocked(x, abits)
                        outs.append(fq.gemm_w6ax_blocked(qb, sa, wp, sw, N, abits))
                    elif it % 4 == 0:
                        outs.append(fq.linear_w6ax(x, wp, sw, N, abits))
                    elif it % 4 == 1:
                        qa, sa = fq.quant_act(x, abits)
                        outs.append(fq.gemm_w6ax(qa, sa, wp, sw, N, abits))
                    elif it % 4 == 3 and abits == 6:  # 6-bit activation storage
                        qp, sa = fq.quant_act_a6_packed(x)
                        outs.append(fq.gemm_w6a6_packed(qp, sa, wp, sw, N))
                    else:  # split-K with one slice: the definition, bit for bit
                        qa, sa = fq.quant_act(x, abits)
                        outs.append(fq.gemm_w6ax_splitk(qa, sa, wp, sw, N, abits, splits=1,
                                                        path=fq.PATH_PREFILL_128X64))
            stream.synchronize()
            results[i] = [o.cpu().numpy().view(np.uint16) for o in outs]
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(CASES))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, case in enumerate(prepared):
        y_ref = case[-1]
        for it, got in enumerate(results[i]):
            bad = np.argwhere(got != y_ref)
            assert bad.size == 0, f"case {CASES[i]} call {it}: {len(bad)} mismatches"
