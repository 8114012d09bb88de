"""GPU parity at the full LLaMA-2 layer sizes, through the same calls the benchmark
times (flexq_pack_w6, flexq_quant_act, flexq_gemm_w6ax with the automatic
decode/prefill choice).

The oracle cannot redo a 4096 x 57344 x 8192 product in a test, but every output
depends only on its own token row and weight row: a sample of rows and 16-column
tiles is quantized and multiplied by the oracle alone and compared bit for bit with
the GPU's outputs at those positions, together with the GPU's activation codes and
scales of the sampled rows and its packed weights and scales of the sampled tiles.
At M = 1 the one-call layer (flexq_linear_w6ax) must also give the two-call result
in full, bit for bit.

Shapes: the toy W6A6 layer, LLaMA-2-7B W6A6 (M 1/16/128), LLaMA-2-13B W6A8
(M 1/64/512), LLaMA-2-70B in W6A6 and W6A8 (M 1/16/64/256/1024/4096), and the
distinct GEMMs of the 80-layer 70B stack (decode M = 32 and prefill M = 2048 in
both precisions; the stack repeats these four layer shapes), and one GPU's share of
the 70B layers under 8-way tensor parallelism.
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

STACK_70B = {"layers": synth.LLAMA2_70B, "M": (32, 2048), "abits": (6, 8)}
# One GPU's share of the 70B layers under 8-way tensor parallelism (qkv and gate_up
# split along N, o and down along K at whole groups): short K loops and narrow N.
TP8_70B = {"layers": {"qkv": (10240 // 8, 8192), "o": (8192, 8192 // 8),
                      "gate_up": (57344 // 8, 8192), "down": (8192, 28672 // 8)},
           "M": (1, 16, 64, 256, 1024, 4096), "abits": (6, 8)}
EXTRA = {"llama2_70b_stack": STACK_70B, "llama2_70b_tp8_shard": TP8_70B}
CASES = []
for wname, wl in list(synth.WORKLOADS.items()) + list(EXTRA.items()):
    for lname in wl["layers"]:
        CASES.append((wname, lname))


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


def sample_rows(M, rng):
    rows = {0, M - 1, M // 2}
    rows.update(int(r) for r in rng.integers(0, M, 3))
    return np.array(sorted(rows))


def sample_tiles(N, rng):
    tiles = {0, N // 16 - 1}
    tiles.update(int(t) for t in rng.integers(0, N // 16, 2))
    return np.array(sorted(tiles))


@pytest.mark.parametrize("wname,lname", CASES, ids=[f"{w}-{l}" for w, l in CASES])
def test_full_size_sampled(fq, wname, lname):
    wl = EXTRA[wname] if wname in EXTRA else synth.WORKLOADS[wname]
    N, K = wl["layers"][lname]
    seed = synth.derive_seed(synth.BASE_SEED, "full", wname, lname)
    rng = np.random.default_rng(seed & 0xFFFFFFFF)
    w = synth.weights(synth.derive_seed(seed, "w"), N, K, nthreads=synth.default_threads())
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))

    tiles = sample_tiles(N, rng)
    cols = np.concatenate([np.arange(16 * t, 16 * t + 16) for t in tiles])
    wp_all = wp.cpu().numpy().view(np.uint32)
    sw_all = sw.cpu().numpy().view(np.uint16)          # [K/128][N]
    # the sampled tiles' packed words and scales against the oracle's packing
    w_s = np.ascontiguousarray(w[cols])
    wp_ref, sw_ref = oracle.pack_w6(w_s)                # tiles in sampled order
    words = 3 * K                                       # one 16-row tile
    for i, t in enumerate(tiles):
        assert np.array_equal(wp_all[t * words:(t + 1) * words], wp_ref[i * words:(i + 1) * words]), \
            f"packed tile {t}"
    assert np.array_equal(sw_all[:, cols].T, sw_ref.view(np.uint16))
    qw_ref, _ = oracle.quant_w6(w_s)
    del w

    for M in wl["M"]:
        x = synth.activations(synth.derive_seed(seed, "x", M), M, K, nthreads=synth.default_threads())
        xd = torch.from_numpy(x).to(DEV)
        rows = sample_rows(M, rng)
        for abits in wl["abits"]:
            say(f"{wname} {lname} M={M} N={N} K={K} abits={abits}")
            qa, sa = fq.quant_act(xd, abits)
            y = fq.gemm_w6ax(qa, sa, wp, sw, N, abits)
            if M == 1:
                y_lin = fq.linear_w6ax(xd, wp, sw, N, abits)
                assert torch.equal(y_lin.view(torch.int16), y.view(torch.int16))
            torch.cuda.synchronize()
            qa_ref, sa_ref = oracle.quant_act(np.ascontiguousarray(x[rows]), abits)
            assert np.array_equal(qa[torch.from_numpy(rows).to(DEV)].cpu().numpy(), qa_ref)
            assert np.array_equal(sa.cpu().numpy()[:, rows].T.view(np.uint32),
                                  sa_ref.view(np.uint32))
            y_ref = oracle.gemm(qa_ref, sa_ref, qw_ref, sw_ref)
            got = y.cpu().numpy()[np.ix_(rows, cols)].view(np.uint16)
            bad = np.argwhere(got != y_ref.view(np.uint16))
            assert bad.size == 0, f"{len(bad)} of {got.size} sampled outputs differ, first " \
                                  f"(row, col) {[(int(rows[i]), int(cols[j])) for i, j in bad[:4]]}"
        del xd
