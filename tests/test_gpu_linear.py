"""GPU parity of flexq_linear_w6ax: one layer from fp16 activations in one call.

For up to 4 rows with rows x K <= 16384 one kernel does both steps (each workgroup
quantizes X into LDS, then streams the weights); otherwise the activation quantizer
and the GEMM run as two kernels with q_a and s_a in the caller's workspace.  Y must
equal, bit for bit, the oracle's chain (quantize, then the group-quantized product)
and the library's own two-call path, for any workspace contents and size at or
above the stated one.

The shapes cover the decode kernel's single and paired 16-column tiles (narrow and
wide N, K beyond 16384), group counts below, at and past the 16 groups a workgroup
folds per round, ragged tile counts, 1 to 5 and 40 rows, and the prefill kernel.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

G = 128
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def u16(t):
    return t.cpu().numpy().view(np.uint16)


def oracle_layer(x, w, abits):
    qa, sa = oracle.quant_act(x, abits)
    wp, sw = oracle.pack_w6(w)
    return oracle.gemm_packed(qa, sa, wp, sw, w.shape[0]).view(np.uint16)


# (M, N, K): 1 to 4 rows on single tiles (N/16 <= 3 x CUs, K <= 16384) and paired
# tiles (wide N with an odd tile count, or K > 16384); group counts 1, 3, 16, 17, 129;
# then 5 and 40 rows (decode kernel) and 300 rows (prefill kernel)
SHAPES = [(1, 16, 128), (2, 48, 384), (3, 208, 2048), (4, 400, 2176), (1, 12304, 256),
          (4, 12304, 384), (2, 64, 16512), (3, 1040, 1024), (5, 48, 1152), (40, 208, 1024),
          (300, 144, 768),
          # the fused quantizer's configurations and its limit: paired tiles on a
          # narrow layer (more than 2 single tiles per CU), rows x K at 16384 exactly and
          # one group past it (two kernels), the largest K it takes at one row and one
          # group past that, a 70B qkv row
          (2, 8320, 1024), (4, 64, 4096), (4, 64, 4224), (1, 64, 16384), (1, 64, 16512),
          (1, 10240, 8192)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("abits", [6, 8])
def test_linear_bit_exact(fq, M, N, K, abits):
    say(f"linear M={M} N={N} K={K} abits={abits}")
    x = synth.activations(synth.derive_seed(31, "x", M, N, K), M, K)
    w = synth.weights(synth.derive_seed(31, "w", M, N, K), N, K)
    wp, sw = fq.pack_w6(to_dev(w))
    xd = to_dev(x)
    y = fq.linear_w6ax(xd, wp, sw, N, abits)
    ref = oracle_layer(x, w, abits)
    got = u16(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    qa, sa = fq.quant_act(xd, abits)
    assert torch.equal(y.view(torch.int16),
                       fq.gemm_w6ax(qa, sa, wp, sw, N, abits).view(torch.int16))


@pytest.mark.parametrize("abits", [6, 8])
def test_linear_quotients_on_rounding_boundaries(fq, abits):
    """Activation groups whose quotients v / s sit exactly on k + 1/2 or one fp16 step
    either side, through the one-call layer 4 rows at a time."""
    qmax = 31 if abits == 6 else 127
    rows = []
    for e in (-4, 0, 3):
        s = 2.0 ** e
        k = np.arange(-qmax, qmax, dtype=np.float64) + 0.5
        ties = (k * s).astype(np.float16)
        for vals in (ties, np.nextafter(ties, np.float16(np.inf)),
                     np.nextafter(ties, np.float16(-np.inf))):
            row = np.zeros(2 * G, dtype=np.float16)
            row[0] = np.float16(qmax * s)
            n = min(len(vals), G - 1)
            row[1:1 + n] = vals[:n]
            row[G] = np.float16(qmax * s)
            row[G + 1:G + 1 + len(vals) - n] = vals[n:]
            rows.append(row)
    x_all = np.stack(rows)
    N = 64
    w = synth.weights(synth.derive_seed(32, "w", abits), N, 2 * G)
    wp, sw = fq.pack_w6(to_dev(w))
    for i in range(0, len(x_all), 4):
        x = np.ascontiguousarray(x_all[i:i + 4])
        y = fq.linear_w6ax(to_dev(x), wp, sw, N, abits)
        assert np.array_equal(u16(y), oracle_layer(x, w, abits)), f"rows {i}..{i + len(x) - 1}"


def test_linear_zero_groups_and_extremes(fq):
    """An all-zero activation row and group (scale 0, codes 0), an all-zero weight
    group, fp16 extremes (65504, subnormals) and a single non-zero per group."""
    M, N, K = 4, 96, 3 * G
    x = synth.activations(synth.derive_seed(33, "x"), M, K)
    w = synth.weights(synth.derive_seed(33, "w"), N, K)
    x[1] = 0
    x[2, G:2 * G] = 0
    x[3, :G] = 0
    x[3, 5] = np.float16(-65504.0)
    x[0, 2 * G:] = np.float16(6e-8)
    x[0, 2 * G + 7] = np.float16(-1e-7)
    w[5, :G] = 0
    for abits in (6, 8):
        wp, sw = fq.pack_w6(to_dev(w))
        y = fq.linear_w6ax(to_dev(x), wp, sw, N, abits)
        assert np.array_equal(u16(y), oracle_layer(x, w, abits))


def test_linear_outputs_guards_and_workspace(fq):
    """Each row count writes exactly its rows (guard bands stay, poison is
    overwritten), also at a 4-byte aligned output; a larger, poisoned workspace is
    accepted and the call repeats bit for bit."""
    N, K = 208, 1024
    w = synth.weights(synth.derive_seed(34, "w"), N, K)
    wp, sw = fq.pack_w6(to_dev(w))
    for M in (1, 2, 3, 4, 6):
        x = synth.activations(synth.derive_seed(34, "x", M), M, K)
        ref = oracle_layer(x, w, 8)
        for off in (0, 2):
            buf = torch.full((M * N + 4096,), -1, dtype=torch.int16, device=DEV)
            y = buf[off:off + M * N].view(torch.float16).view(M, N)
            need = fq.linear_w6ax_workspace_bytes(M, K)
            assert need >= M * K + M * (K // G) * 4
            ws = torch.full((need + 512,), 0xAB, dtype=torch.uint8, device=DEV)
            for _ in range(2):
                fq.linear_w6ax(to_dev(x), wp, sw, N, 8, y=y, workspace=ws)
                assert np.array_equal(u16(y), ref), f"M={M} offset={off}"
            assert torch.all(buf[:off] == -1) and torch.all(buf[off + M * N:] == -1)


def test_linear_rejects_bad_arguments_before_launch(fq):
    N, K = 32, 256
    w = synth.weights(synth.derive_seed(35, "w"), N, K)
    wp, sw = fq.pack_w6(to_dev(w))
    x = to_dev(synth.activations(synth.derive_seed(35, "x"), 8, K))
    # a workspace that is too small is refused by the binding (the C ABI refuses it
    # too: the ctypes tests of the ABI call it directly)
    with pytest.raises(ValueError, match="workspace"):
        fq.linear_w6ax(x, wp, sw, N, 8,
                       workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    xu = torch.empty(2 * K + 4, dtype=torch.float16, device=DEV)[4:].view(2, K)  # 8 B past
    assert xu.data_ptr() % 16 == 8
    with pytest.raises(fq.FlexqError, match="UNSUPPORTED"):
        fq.linear_w6ax(xu, wp, sw, N, 6)
    with pytest.raises(fq.FlexqError, match="INVALID"):
        fq.linear_w6ax(x[:2], wp, sw, N, 7)
