"""GPU parity on seeded random shapes: every entry point, kernel and prefill tile on
shapes drawn to land on and around their boundaries.

Each case draws M from 1 to 384 (decode passes of 16/32/48/64 rows, prefill row
tiles of 64, 128 and 256, ragged tails), N a multiple of 16 up to 2560 (8192 for a
quarter of the cases), K a multiple of 128 up to 32 groups (128 for that quarter),
the activation precision, the path (automatic, decode, automatic prefill tile, one
named tile, the warp-specialized kernel or the 64 x 128 tile) and the value
distribution (the standard synthetic X and W; every third token row and the first
group of every weight row zero; magnitudes near the fp16 top; magnitudes that give
subnormal fp16 weight scales).  Per case, against the oracle:

* packed weights and their scales, activation codes and scales bit for bit;
* Y bit for bit from the automatic path and the drawn path, the blocked-code pair
  (flexq_quant_act_blocked, flexq_gemm_w6ax_blocked), for A6 the packed pair
  (flexq_quant_act_a6_packed, flexq_gemm_w6a6_packed), the one-call layer and, where
  its codes fit the library's array, the allocation-free layer;
* the split-K GEMM with a drawn slice count and tile: within the tolerance module's
  bound, and the same bits on a second call.

FLEXQ_RANDOM_CASES and FLEXQ_RANDOM_SEED widen a run (default 48 cases, seed 51).
"""
import os

import numpy as np
import pytest

import oracle
import synth
import tolerance

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
G = 128
N_CASES = int(os.environ.get("FLEXQ_RANDOM_CASES", "48"))
SEED = int(os.environ.get("FLEXQ_RANDOM_SEED", "51"))
M_CHOICES = [1, 2, 3, 4, 5, 6, 8, 9, 12, 15, 16, 17, 20, 24, 31, 32, 33, 40, 47, 48, 49, 56,
             63, 64, 65, 80, 96, 127, 128, 129, 160, 192, 255, 256, 257, 300, 320, 384]
DIST_NAMES = ("synthetic", "zero rows and groups", "near fp16 max", "subnormal scales")


def draw_cases():
    rng = np.random.default_rng(synth.derive_seed(SEED, "shapes") & 0xFFFFFFFF)
    cases = []
    for i in range(N_CASES):
        M = int(rng.choice(M_CHOICES))
        big = int(rng.integers(0, 4)) == 0
        N = 16 * int(rng.integers(1, 513 if big else 161))
        K = G * int(rng.integers(1, 129 if big else 33))
        abits = int(rng.choice([6, 8]))
        path = int(rng.integers(0, 8))
        dist = int(rng.integers(0, 4))
        splits = int(rng.integers(0, min(K // G, 8) + 1))   # 0: the planned count
        tile = int(rng.choice([2, 3, 4, 5, 7]))              # prefill auto or a named tile
        cases.append((i, M, N, K, abits, path, dist, splits, tile))
    return cases


CASES = draw_cases()


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def operands(i, M, N, K, dist):
    """fp16 X[M][K] and W[N][K] of case i in the drawn value distribution."""
    x = synth.activations(synth.derive_seed(SEED, "x", i), M, K)
    w = synth.weights(synth.derive_seed(SEED, "w", i), N, K)
    if dist == 1:
        x[::3, :] = 0
        w[:, :G] = 0
    elif dist == 2:
        x = (x.astype(np.float32) * 3000).clip(-65504, 65504).astype(np.float16)
        w = (w.astype(np.float32) * 1000).clip(-65504, 65504).astype(np.float16)
    elif dist == 3:
        x = (x.astype(np.float32) * 1e-4).astype(np.float16)
        w = (w.astype(np.float32) * 1e-3).astype(np.float16)
    return x, w


def bits16(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("i,M,N,K,abits,path,dist,splits,tile", CASES,
                         ids=[f"{c[0]}-M{c[1]}-N{c[2]}-K{c[3]}-a{c[4]}-p{c[5]}-d{c[6]}"
                              for c in CASES])
def test_random_shape_bit_exact(fq, i, M, N, K, abits, path, dist, splits, tile):
    print(f"case {i}: M={M} N={N} K={K} abits={abits} path={path} "
          f"dist={DIST_NAMES[dist]} splits={splits} tile={tile}", flush=True)
    x, w = operands(i, M, N, K, dist)
    qa_ref, sa_ref = oracle.quant_act(x, abits)
    wp_ref, sw_ref = oracle.pack_w6(w)
    y_ref, acc_ref, S_ref = oracle.gemm_packed(qa_ref, sa_ref, wp_ref, sw_ref, N, want_acc=True)
    y_ref = y_ref.view(np.uint16)
    xd = torch.from_numpy(x).to(DEV)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    assert np.array_equal(wp.cpu().numpy().view(np.uint32), wp_ref.view(np.uint32))
    assert np.array_equal(sw.cpu().numpy().T.view(np.uint16), sw_ref.view(np.uint16))
    qa, sa = fq.quant_act(xd, abits)
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().T.view(np.uint32), sa_ref.view(np.uint32))
    for p in sorted({fq.PATH_AUTO, path}):
        got = bits16(fq.gemm_w6ax(qa, sa, wp, sw, N, abits, path=p))
        bad = np.argwhere(got != y_ref)
        assert bad.size == 0, f"path {p}: {len(bad)} mismatches, first at {bad[:4].tolist()}"
    # codes in 16-row blocks: the oracle's blocking and the same Y
    qb, sab = fq.quant_act_blocked(xd, abits)
    assert np.array_equal(qb.cpu().numpy(), oracle.block_act(qa_ref))
    assert torch.equal(sab.view(torch.int32), sa.view(torch.int32))
    assert np.array_equal(bits16(fq.gemm_w6ax_blocked(qb, sab, wp, sw, N, abits)), y_ref)
    if abits == 6:  # 6-bit activation storage: the oracle's packing and the same Y
        qp, sap = fq.quant_act_a6_packed(xd)
        assert np.array_equal(qp.cpu().numpy().view(np.uint32), oracle.pack_act_a6(qa_ref))
        assert torch.equal(sap.view(torch.int32), sa.view(torch.int32))
        assert np.array_equal(bits16(fq.gemm_w6a6_packed(qp, sap, wp, sw, N)), y_ref)
    # the one-call layers
    assert np.array_equal(bits16(fq.linear_w6ax(xd, wp, sw, N, abits)), y_ref)
    if fq.linear_w6ax_workspace_bytes(M, K) <= fq.NOALLOC_SCRATCH_BYTES:
        yn = torch.empty((M, N), dtype=torch.float16, device=DEV)
        fq.linear_w6ax_noalloc(xd, wp, sw, N, abits, yn)
        assert np.array_equal(bits16(yn), y_ref)
    # split-K: within the tolerance, and the same bits twice
    acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y1 = fq.gemm_w6ax_splitk(qa, sa, wp, sw, N, abits, splits=splits, path=tile, acc=acc)
    y2 = fq.gemm_w6ax_splitk(qa, sa, wp, sw, N, abits, splits=splits, path=tile)
    ok, n_ulp, n_acc = tolerance.check(bits16(y1), y_ref, acc.cpu().numpy(), acc_ref, S_ref)
    assert ok, f"split-K S={splits} tile={tile}: {n_ulp} beyond one ulp, {n_acc} beyond the bound"
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
