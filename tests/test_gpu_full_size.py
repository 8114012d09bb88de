"""GPU parity at the full LLaMA-2 layer sizes, through the same calls the benchmark
times (flexq_pack_w6, flexq_quant_act, flexq_gemm_w6ax with the automatic
decode/prefill choice), against the CPU oracle on the same seeded inputs.

Scope, for every layer of every workload:

* packed weights and weight scales: the whole tensor, bit for bit;
* activation codes and activation scales at every token count: the whole tensor;
* Y: the whole output for the toy layer, every LLaMA-2-7B shape and every shape
  with M <= 64 (the decode kernel's range); at larger M every column of 4 rows
  (first, last, two seeded) plus 4096 seeded (row, column) outputs spread over the
  whole grid of prefill tiles;
* the int32 group dots (flexq_gemm_w6ax_group_dots): a slab of 16 token rows x 64
  weight rows (four 16-row tiles) x every group, at every token count.

Y is compared bit for bit: both kernels keep the sequential ascending-group fp32
order of the definition.  Where the split-K plan cuts K into slices (mid-sized M on
narrow layers), flexq_gemm_w6ax_splitk runs in the planned configuration too and its
whole Y and fp32 accumulator are checked against the tolerance for a changed
summation order (tests/tolerance.py).  At M <= 64 the one-call layer (flexq_linear_w6ax) must
also give the two-call result in full, the codes in 16-row blocks
(flexq_quant_act_blocked) and the streaming GEMM over them (flexq_gemm_w6ax_blocked)
are checked whole against the oracle's blocking and Y, and for A6 so are the packed
activations (flexq_quant_act_a6_packed) and the GEMM over them (flexq_gemm_w6a6_packed).

Workloads: the toy W6A6 layer, LLaMA-2-7B W6A6 (M 1/16/128), LLaMA-2-13B W6A8
(M 1/64/512), LLaMA-2-70B in W6A6 and W6A8 (M 1/16/64/256/1024/4096), the distinct
GEMMs of the 80-layer 70B stack (decode M = 32 and prefill M = 2048 in both
precisions; every layer of the stack holds the same four shapes and, in the
benchmark, the same synthetic values), and one GPU's share of the 70B layers under
8-way tensor parallelism.  The oracle's quantizers run over row blocks in parallel
threads and its GEMM over column blocks, so each case finishes in seconds.
"""
from concurrent.futures import ThreadPoolExecutor

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
FULL_Y_MAX_M = 64
PAIRS = 4096

STACK_70B = {"layers": synth.LLAMA2_70B, "M": (32, 2048), "abits": (6, 8)}
# One GPU's share of the 70B layers under 8-way tensor parallelism (qkv and gate_up
# split along N, o and down along K at whole groups): short K loops and narrow N.
TP8_70B = {"layers": {"qkv": (10240 // 8, 8192), "o": (8192, 8192 // 8),
                      "gate_up": (57344 // 8, 8192), "down": (8192, 28672 // 8)},
           "M": (1, 16, 64, 256, 1024, 4096), "abits": (6, 8)}
EXTRA = {"llama2_70b_stack": STACK_70B, "llama2_70b_tp8_shard": TP8_70B}
FULL_Y_WORKLOADS = {"toy_w6a6", "llama2_7b_w6a6"}
CASES = []
for wname, wl in list(synth.WORKLOADS.items()) + list(EXTRA.items()):
    for lname in wl["layers"]:
        CASES.append((wname, lname))

THREADS = synth.default_threads()
_pool = ThreadPoolExecutor(THREADS)


@pytest.fixture(scope="module")
def fq():
    import w6a6_w6a8_integer_amd as fq
    fq.lib()
    return fq


def say(*a):
    print(*a, flush=True)


def _blocks(n, step=1):
    """Split range(n) into up to 2 * THREADS blocks whose bounds are multiples of step."""
    per = max(step, -(-n // (2 * THREADS) // step) * step)
    return [(a, min(n, a + per)) for a in range(0, n, per)]


def oracle_quant_w6(w):
    N, K = w.shape
    qw = np.empty((N, K), np.int8)
    sw = np.empty((N, K // G), np.float16)

    def job(ab):
        a, b = ab
        qw[a:b], sw[a:b] = oracle.quant_w6(w[a:b])
    list(_pool.map(job, _blocks(N)))
    return qw, sw


def oracle_pack_codes(qw):
    N, K = qw.shape
    wp = np.empty(3 * N * K // 16, np.uint32)

    def job(ab):   # rows a..b are 16-row tiles a/16..b/16, a contiguous run of words
        a, b = ab
        wp[3 * a * K // 16:3 * b * K // 16] = oracle.pack_codes(qw[a:b])
    list(_pool.map(job, _blocks(N, 16)))
    return wp


def oracle_quant_act(x, abits):
    M, K = x.shape
    qa = np.empty((M, K), np.int8)
    sa = np.empty((M, K // G), np.float32)

    def job(ab):
        a, b = ab
        qa[a:b], sa[a:b] = oracle.quant_act(x[a:b], abits)
    list(_pool.map(job, _blocks(M)))
    return qa, sa


def first_diffs(got, ref, index):
    bad = np.argwhere(got != ref)
    return f"{len(bad)} of {got.size} differ, first at {[index(b) for b in bad[:4]]}"


@pytest.mark.parametrize("wname,lname", CASES, ids=[f"{w}-{l}" for w, l in CASES])
def test_full_size(fq, wname, lname):
    wl = EXTRA[wname] if wname in EXTRA else synth.WORKLOADS[wname]
    N, K = wl["layers"][lname]
    seed = synth.derive_seed(synth.BASE_SEED, "full", wname, lname)
    rng = np.random.default_rng(seed & 0xFFFFFFFF)
    say(f"{wname} {lname}: N={N} K={K}: pack_w6")
    w = synth.weights(synth.derive_seed(seed, "w"), N, K, nthreads=THREADS)
    wp, sw = fq.pack_w6(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()

    # packed weights and weight scales, whole tensors
    qw, sw_ref = oracle_quant_w6(w)
    del w
    wp_ref = oracle_pack_codes(qw)
    wp_got = wp.cpu().numpy().view(np.uint32)[:wp_ref.size]
    assert np.array_equal(wp_got, wp_ref), first_diffs(
        wp_got, wp_ref, lambda b: f"dword {int(b[0])} (tile {int(b[0]) // (3 * K)})")
    sw_got = sw.cpu().numpy().view(np.uint16).T          # group-major -> [N][G]
    assert np.array_equal(sw_got, sw_ref.view(np.uint16)), first_diffs(
        sw_got, sw_ref.view(np.uint16), lambda b: (int(b[0]), int(b[1])))
    del wp_got, wp_ref

    for M in wl["M"]:
        x = synth.activations(synth.derive_seed(seed, "x", M), M, K, nthreads=THREADS)
        xd = torch.from_numpy(x).to(DEV)
        for abits in wl["abits"]:
            say(f"{wname} {lname}: M={M} N={N} K={K} abits={abits}")
            qa, sa = fq.quant_act(xd, abits)
            y = fq.gemm_w6ax(qa, sa, wp, sw, N, abits)
            torch.cuda.synchronize()

            # activation codes and scales, whole tensors
            qa_ref, sa_ref = oracle_quant_act(x, abits)
            qa_got = qa.cpu().numpy()
            assert np.array_equal(qa_got, qa_ref), first_diffs(
                qa_got, qa_ref, lambda b: (int(b[0]), int(b[1])))
            sa_got = sa.cpu().numpy().T.view(np.uint32)
            assert np.array_equal(sa_got, sa_ref.view(np.uint32)), first_diffs(
                sa_got, sa_ref.view(np.uint32), lambda b: (int(b[0]), int(b[1])))
            del qa_got, sa_got

            # group dots: 16 token rows x 64 weight rows x every group
            rows16 = np.sort(rng.choice(M, min(M, 16), replace=False))
            t0 = int(rng.integers(0, max(1, N // 16 - 3)))
            nt = min(4, N // 16 - t0)
            dots = fq.gemm_w6ax_group_dots(
                qa[torch.from_numpy(rows16).to(DEV)].contiguous(),
                wp[3 * K * t0:3 * K * (t0 + nt)], 16 * nt)
            torch.cuda.synchronize()
            d_ref = oracle.group_dots(np.ascontiguousarray(qa_ref[rows16]),
                                      np.ascontiguousarray(qw[16 * t0:16 * (t0 + nt)]),
                                      nthreads=THREADS)
            d_got = dots.cpu().numpy()
            assert np.array_equal(d_got, d_ref), first_diffs(
                d_got, d_ref, lambda b: (int(rows16[b[0]]), 16 * t0 + int(b[1]), int(b[2])))

            # Y
            full = None   # the oracle's whole (Y, fp32 accumulator, S), computed once
            if M <= FULL_Y_MAX_M or wname in FULL_Y_WORKLOADS:
                full = oracle.gemm(qa_ref, sa_ref, qw, sw_ref, nthreads=THREADS, want_acc=True)
                y_ref = full[0]
                y_got = y.cpu().numpy().view(np.uint16)
                assert np.array_equal(y_got, y_ref.view(np.uint16)), first_diffs(
                    y_got, y_ref.view(np.uint16), lambda b: (int(b[0]), int(b[1])))
                if M <= FULL_Y_MAX_M:
                    y_lin = fq.linear_w6ax(xd, wp, sw, N, abits)
                    assert torch.equal(y_lin.view(torch.int16), y.view(torch.int16))
                if M <= FULL_Y_MAX_M:
                    # codes in 16-row blocks: the whole blocked tensor, and the whole Y of
                    # the streaming kernel over it
                    say(f"{wname} {lname}: M={M} abits={abits}: blocked activation codes")
                    qb, sab = fq.quant_act_blocked(xd, abits)
                    yb = fq.gemm_w6ax_blocked(qb, sab, wp, sw, N, abits)
                    torch.cuda.synchronize()
                    assert np.array_equal(qb.cpu().numpy(), oracle.block_act(qa_ref))
                    assert torch.equal(sab.view(torch.int32), sa.view(torch.int32))
                    yb_got = yb.cpu().numpy().view(np.uint16)
                    assert np.array_equal(yb_got, y_ref.view(np.uint16)), first_diffs(
                        yb_got, y_ref.view(np.uint16), lambda b: (int(b[0]), int(b[1])))
                    del qb, sab, yb
                if M <= FULL_Y_MAX_M and abits == 6:
                    # 6-bit activation storage: the whole packed tensor, and the whole Y
                    # of the streaming kernel over it
                    say(f"{wname} {lname}: M={M}: packed A6 activations")
                    qp, sap = fq.quant_act_a6_packed(xd)
                    yp = fq.gemm_w6a6_packed(qp, sap, wp, sw, N)
                    torch.cuda.synchronize()
                    qp_ref = oracle.pack_act_a6(qa_ref)
                    qp_got = qp.cpu().numpy().view(np.uint32)
                    assert np.array_equal(qp_got, qp_ref), first_diffs(
                        qp_got, qp_ref, lambda b: (int(b[0]), int(b[1]) // 3))
                    assert torch.equal(sap.view(torch.int32), sa.view(torch.int32))
                    yp_got = yp.cpu().numpy().view(np.uint16)
                    assert np.array_equal(yp_got, y_ref.view(np.uint16)), first_diffs(
                        yp_got, y_ref.view(np.uint16), lambda b: (int(b[0]), int(b[1])))
                    del qp, sap, yp
            else:
                rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 2)]))
                y_ref = oracle.gemm(np.ascontiguousarray(qa_ref[rows]),
                                    np.ascontiguousarray(sa_ref[rows]), qw, sw_ref,
                                    nthreads=THREADS)
                y_got = y[torch.from_numpy(rows).to(DEV)].cpu().numpy().view(np.uint16)
                assert np.array_equal(y_got, y_ref.view(np.uint16)), first_diffs(
                    y_got, y_ref.view(np.uint16), lambda b: (int(rows[b[0]]), int(b[1])))
                pm = rng.integers(0, M, PAIRS)
                pn = rng.integers(0, N, PAIRS)
                got = y[torch.from_numpy(pm).to(DEV), torch.from_numpy(pn).to(DEV)]
                got = got.cpu().numpy().view(np.uint16)

                def one(i):
                    m, n = int(pm[i]), int(pn[i])
                    return oracle.gemm(qa_ref[m:m + 1], sa_ref[m:m + 1], qw[n:n + 1],
                                       sw_ref[n:n + 1], nthreads=1).view(np.uint16)[0, 0]
                ref = np.array(list(_pool.map(one, range(PAIRS))), np.uint16)
                assert np.array_equal(got, ref), first_diffs(
                    got, ref, lambda b: (int(pm[b[0]]), int(pn[b[0]])))

            # split-K where the plan splits (as the benchmark runs it): the whole Y and
            # fp32 accumulator within the tolerance of the sequential definition
            S_plan, tile = fq.splitk_plan(M, N, K)
            if S_plan > 1:
                say(f"{wname} {lname}: M={M} abits={abits}: split-K S={S_plan} tile path {tile}")
                acc = torch.empty((M, N), dtype=torch.float32, device=DEV)
                ys = fq.gemm_w6ax_splitk(qa, sa, wp, sw, N, abits, acc=acc)
                torch.cuda.synchronize()
                if full is None:
                    full = oracle.gemm(qa_ref, sa_ref, qw, sw_ref, nthreads=THREADS,
                                       want_acc=True)
                ok, n_ulp, n_acc = tolerance.check(ys.cpu().numpy().view(np.uint16),
                                                   full[0].view(np.uint16), acc.cpu().numpy(),
                                                   full[1], full[2])
                assert ok and n_acc == 0, (n_ulp, n_acc)
                del ys, acc
            del y, full
        del xd
