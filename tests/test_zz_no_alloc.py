"""flexq_linear_w6ax_noalloc, the one-call layer that allocates nothing (its
activation codes and scales go to the library's own per-GPU device array), called
through the C ABI and checked bit for bit against flexq_linear_w6ax, the entry point
with a caller workspace, on consecutive calls of decreasing size (each call reuses
the array the previous one filled), and against the CPU oracle."""
import ctypes

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    import w6a6_w6a8_integer_amd as fq
    lib = fq.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # decreasing scratch use: the prefill kernel, then the decode kernel, then a tiny layer
    cases = [(300, 384, 1024, 8), (40, 512, 2048, 6), (3, 256, 512, 8)]
    for M, N, K, abits in cases:
        say(f"noalloc M={M} N={N} K={K} abits={abits}")
        x = synth.activations(synth.derive_seed(91, "x", M, N, K), M, K)
        w = synth.weights(synth.derive_seed(91, "w", M, N, K), N, K)
        xd = torch.from_numpy(x).to(DEV)
        wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
        y_ws = fq.linear_w6ax(xd, wp, sw, N, abits)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        rc = lib.flexq_linear_w6ax_noalloc(
            ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(wp.data_ptr()),
            ctypes.c_void_p(sw.data_ptr()), M, N, K, 128, abits, ctypes.c_void_p(y.data_ptr()),
            ctypes.c_void_p(stream))
        assert rc == 0, fq.lib().flexq_status_string(rc)
        torch.cuda.synchronize()
        got = y.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, y_ws.cpu().numpy().view(np.uint16)), (M, N, K)
        qa, sa = oracle.quant_act(x, abits)
        wp_ref, sw_ref = oracle.pack_w6(w)
        assert np.array_equal(got, oracle.gemm_packed(qa, sa, wp_ref, sw_ref, N).view(np.uint16))
        # the binding's wrapper of the same entry point
        y2 = fq.linear_w6ax_noalloc(xd, wp, sw, N, abits, torch.empty_like(y))
        assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


def test_noalloc_refuses_shapes_beyond_its_array_before_any_launch():
    import w6a6_w6a8_integer_amd as fq
    K = 28672
    M = fq.NOALLOC_SCRATCH_BYTES // K          # a little more than the array holds
    assert fq.linear_w6ax_workspace_bytes(M, K) > fq.NOALLOC_SCRATCH_BYTES
    assert fq.linear_w6ax_workspace_bytes(2269, K) <= fq.NOALLOC_SCRATCH_BYTES
    x = torch.empty((M, K), dtype=torch.float16, device=DEV)
    wp = torch.empty(3 * 16 * K // 16, dtype=torch.int32, device=DEV)
    sw = torch.empty((K // 128, 16), dtype=torch.float16, device=DEV)
    y = torch.full((M, 16), 1.0, dtype=torch.float16, device=DEV)
    with pytest.raises(fq.FlexqError, match="UNSUPPORTED"):
        fq.linear_w6ax_noalloc(x, wp, sw, 16, 6, y)
    torch.cuda.synchronize()
    assert torch.all(y == 1.0)                 # nothing ran
