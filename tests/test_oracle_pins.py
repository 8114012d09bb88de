"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a library routine (numpy), exact rational
arithmetic (fractions), a closed form, an invariant the method guarantees, or a
hand-derived fixture under tests/golden/.  None of them call the GPU library.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
G = 128


def f16(vals):
    return np.asarray(vals, dtype=np.float16)


def bits16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# binary16 conversions against numpy (library routine)
# ---------------------------------------------------------------------------

def test_f16_widening_matches_numpy_all_patterns():
    lib = oracle._load()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([lib.oracle_f16_to_f32(int(p)) for p in pats], dtype=np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f32_to_f16_rounding_matches_numpy():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(5000) * 1e-5).astype(np.float32),   # fp16 subnormal range
        (rng.standard_normal(5000) * 3e4).astype(np.float32),    # near overflow
        # exact ties between two fp16 neighbours (normal and subnormal)
        (np.arange(1, 2000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10),
        (np.arange(1, 500, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24),
        np.array([65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0],
                 np.float32),
    ])
    lib = oracle._load()
    got = np.array([lib.oracle_f32_to_f16(float(v)) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# packed 6-bit format
# ---------------------------------------------------------------------------

def _golden_units():
    rows = []
    with open(os.path.join(GOLDEN, "pack_units.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            codes, words = line.split(";")
            rows.append(([int(c) for c in codes.split()], [int(w, 16) for w in words.split()]))
    return rows


@pytest.mark.parametrize("codes,words", _golden_units())
def test_pack_unit_golden(codes, words):
    assert [int(x) for x in oracle.pack_unit(codes)] == words
    assert [int(x) for x in oracle.unpack_unit(words)] == codes


def test_pack_unit_round_trip_every_code_every_position():
    rng = np.random.default_rng(1)
    for pos in range(16):
        for code in range(-32, 32):
            q = rng.integers(-32, 32, 16).astype(np.int8)
            q[pos] = code
            assert np.array_equal(oracle.unpack_unit(oracle.pack_unit(q)), q)
    for _ in range(2000):
        q = rng.integers(-32, 32, 16).astype(np.int8)
        assert np.array_equal(oracle.unpack_unit(oracle.pack_unit(q)), q)


def test_pack_unit_each_code_bit_owns_one_packed_bit():
    """96 code bits map one to one onto the 96 bits of the 3 dwords."""
    seen = set()
    for pos in range(16):
        for b in range(6):
            q = np.zeros(16, np.int8)
            v = 1 << b
            q[pos] = v - 64 if v >= 32 else v
            d = oracle.pack_unit(q)
            ones = [(w, i) for w in range(3) for i in range(32) if (int(d[w]) >> i) & 1]
            assert len(ones) == 1, (pos, b, ones)
            assert ones[0] not in seen
            seen.add(ones[0])
    assert len(seen) == 96


def test_unit_offset_is_a_bijection_and_tiles_are_contiguous():
    for N, K in [(16, 16), (32, 128), (48, 256)]:
        offs = sorted(oracle.unit_offset(n, u, K) for n in range(N) for u in range(K // 16))
        assert offs == list(range(0, 3 * N * K // 16, 3))
        # all units of one 16-row tile occupy one contiguous block of K*12 bytes
        for t in range(N // 16):
            block = {oracle.unit_offset(n, u, K) // 3 for n in range(16 * t, 16 * t + 16)
                     for u in range(K // 16)}
            assert block == set(range(t * K, (t + 1) * K))
        # the 64 lanes of one 64-deep k-chunk of a tile read 64 consecutive units
        base = oracle.unit_offset(0, 0, K)
        lanes = [oracle.unit_offset(l % 16, l // 16, K) for l in range(64)]
        assert lanes == [base + 3 * l for l in range(64)]


def test_pack_codes_matrix_round_trip():
    rng = np.random.default_rng(3)
    q = rng.integers(-32, 32, (48, 384)).astype(np.int8)
    wp = oracle.pack_codes(q)
    assert wp.size == 48 * 384 * 3 // 16
    assert np.array_equal(oracle.unpack_codes(wp, 48, 384), q)


# ---------------------------------------------------------------------------
# 6-bit activation storage: the packed unit, row by row
# ---------------------------------------------------------------------------

def test_pack_act_a6_golden_units_in_row_order():
    """A 2 x 48 code matrix built from the hand-derived units: unit u of row m is
    golden line (3m + u) % 6 and must sit, as those three words, at dword
    3 * (3m + u) (row-major units, 0.75 K bytes per row)."""
    units = _golden_units()
    M, K = 2, 48
    qa = np.zeros((M, K), np.int8)
    for m in range(M):
        for u in range(K // 16):
            qa[m, 16 * u:16 * u + 16] = units[(3 * m + u) % len(units)][0]
    qp = oracle.pack_act_a6(qa)
    assert qp.shape == (M, 3 * K // 16) and qp.nbytes == M * K * 3 // 4
    flat = qp.reshape(-1)
    for m in range(M):
        for u in range(K // 16):
            words = units[(3 * m + u) % len(units)][1]
            assert [int(w) for w in flat[3 * (3 * m + u):3 * (3 * m + u) + 3]] == words
    assert np.array_equal(oracle.unpack_act_a6(qp, K), qa)


def test_pack_act_a6_is_the_weight_unit_grid_transposed():
    """For one 16-row block the packed weights (pinned above) hold unit (n, u) at
    unit index 16u + n; the activation layout holds unit (m, u) at m * K/16 + u:
    the same units, the grid transposed."""
    rng = np.random.default_rng(11)
    K = 384
    q = rng.integers(-32, 32, (16, K)).astype(np.int8)
    act = oracle.pack_act_a6(q).reshape(16, K // 16, 3)
    wts = oracle.pack_codes(q).reshape(K // 16, 16, 3).transpose(1, 0, 2)
    assert np.array_equal(act, wts)


def test_pack_act_a6_one_code_touches_one_unit():
    M, K = 3, 256
    base = oracle.pack_act_a6(np.zeros((M, K), np.int8)).reshape(-1)
    assert not base.any()
    for m, k, code in [(0, 0, 1), (1, 17, -32), (2, 255, 31), (2, 128, -1)]:
        qa = np.zeros((M, K), np.int8)
        qa[m, k] = code
        d = oracle.pack_act_a6(qa).reshape(-1)
        changed = sorted({int(i) // 3 for i in np.flatnonzero(d)})
        assert changed == [m * (K // 16) + k // 16]


def test_pack_act_a6_round_trip_and_range():
    rng = np.random.default_rng(12)
    qa = rng.integers(-32, 32, (5, 1152)).astype(np.int8)
    assert np.array_equal(oracle.unpack_act_a6(oracle.pack_act_a6(qa), 1152), qa)
    # the A6 quantizer's codes (|q| <= 31) always fit; A8 codes beyond 6 bits do not
    x = synth.activations(synth.derive_seed(synth.BASE_SEED, "a6pin"), 4, 512)
    qa6, _ = oracle.quant_act(x, 6)
    assert np.array_equal(oracle.unpack_act_a6(oracle.pack_act_a6(qa6), 512), qa6)
    for bad in (32, -33, 127, -127):
        q = np.zeros((1, 16), np.int8)
        q[0, 3] = bad
        try:
            oracle.pack_act_a6(q)
        except ValueError:
            continue
        raise AssertionError(f"code {bad} does not fit 6 bits but was packed")


# ---------------------------------------------------------------------------
# activation codes in 16-row blocks (a layout: pinned to numpy and by hand)
# ---------------------------------------------------------------------------

def test_block_act_is_the_padded_reshape():
    """The blocked layout equals numpy's view of the zero-padded [M][K] codes as
    [block][row][group][half][byte] with the row axis moved inside the half."""
    rng = np.random.default_rng(13)
    for M, K in [(1, 128), (16, 256), (20, 384), (33, 1152)]:
        qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
        Mp = (M + 15) // 16 * 16
        pad = np.zeros((Mp, K), np.int8)
        pad[:M] = qa
        ref = pad.reshape(Mp // 16, 16, K // 128, 2, 64).transpose(0, 2, 3, 1, 4).reshape(-1)
        blk = oracle.block_act(qa)
        assert np.array_equal(blk, ref)
        assert np.array_equal(oracle.unblock_act(blk, M, K), qa)


def test_block_act_places_one_code_by_hand():
    # row 17, column 200 of a 20 x 256 matrix: block 1, row 1 in it, group 1, second
    # half of the group (200 - 128 = 72 >= 64), byte 8 of it:
    # 1*16*256 + 1*2048 + 1*1024 + 1*64 + 8 = 7240
    qa = np.zeros((20, 256), np.int8)
    qa[17, 200] = -77
    blk = oracle.block_act(qa)
    assert blk.size == 32 * 256
    assert np.flatnonzero(blk).tolist() == [7240] and blk[7240] == -77
    qa[:] = 5                                # every real code; the 12 pad rows stay zero
    blk = oracle.block_act(qa)
    assert int(np.count_nonzero(blk)) == 20 * 256


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def _golden_ties():
    rows = []
    with open(os.path.join(GOLDEN, "quant_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, xs, s, qs = line.split(";")
            rows.append((int(a), [float(v) for v in xs.split()], float(s),
                         [int(v) for v in qs.split()]))
    return rows


@pytest.mark.parametrize("abits,xs,scale,codes", _golden_ties())
def test_quant_act_ties_reduce_to_round_half_even(abits, xs, scale, codes):
    x = np.zeros((1, G), np.float16)
    x[0, :len(xs)] = xs
    qa, sa = oracle.quant_act(x, abits)
    assert sa[0, 0] == scale
    assert list(qa[0, :len(codes)]) == codes
    # the same reduction holds against Python's round(), which rounds half to even
    assert list(qa[0, :len(xs)]) == [round(v) for v in xs]
    assert not qa[0, len(xs):].any()


def test_quant_w6_ties_reduce_to_round_half_even():
    xs = [31.0, 0.5, 1.5, 2.5, -0.5, -2.5, 30.5, -29.5, 7.5, 8.5]
    w = np.zeros((1, G), np.float16)
    w[0, :len(xs)] = xs
    qw, sw = oracle.quant_w6(w)
    assert float(sw[0, 0]) == 1.0
    assert list(qw[0, :len(xs)]) == [round(v) for v in xs]


def _exact_round_half_even(fr: Fraction) -> int:
    return round(fr)   # Fraction.__round__ rounds half to even


def _near_tie(fr: Fraction, tol=Fraction(1, 1 << 18)) -> bool:
    return abs((fr - Fraction(1, 2)) - round(fr - Fraction(1, 2))) < tol


@pytest.mark.parametrize("abits", [6, 8])
def test_quant_act_matches_exact_rational_rounding(abits):
    """q = round_half_even(x / s) computed in exact rationals, with s the fp32
    IEEE quotient amax / qmax taken from numpy (a library routine)."""
    qmax = 31 if abits == 6 else 127
    x = synth.activations(synth.derive_seed(11, abits), 6, 4 * G)
    qa, sa = oracle.quant_act(x, abits)
    checked = 0
    for m in range(x.shape[0]):
        for g in range(4):
            grp = x[m, g * G:(g + 1) * G].astype(np.float32)
            amax = np.max(np.abs(grp))
            s = np.float32(amax) / np.float32(qmax)        # IEEE binary32 division
            assert sa[m, g] == s
            for i in range(G):
                quo = Fraction(float(grp[i])) / Fraction(float(s))
                if _near_tie(quo):
                    # the binary32 quotient may land on the tie: numpy's IEEE
                    # division and rint decide it
                    q = int(np.rint(grp[i] / s))
                else:
                    q = _exact_round_half_even(quo)
                    checked += 1
                assert qa[m, g * G + i] == max(-qmax, min(qmax, q))
    assert checked > 0.99 * 6 * 4 * G


def test_quant_w6_matches_exact_rational_rounding():
    w = synth.weights(synth.derive_seed(12), 8, 4 * G)
    qw, sw = oracle.quant_w6(w)
    for n in range(8):
        for g in range(4):
            grp = w[n, g * G:(g + 1) * G].astype(np.float32)
            amax = np.max(np.abs(grp))
            s16 = (np.float32(amax) / np.float32(31)).astype(np.float16)  # IEEE div, then RNE
            assert sw[n, g].view(np.uint16) == s16.view(np.uint16)
            for i in range(G):
                quo = Fraction(float(grp[i])) / Fraction(float(s16))
                if _near_tie(quo):
                    q = int(np.rint(grp[i] / np.float32(s16)))
                else:
                    q = _exact_round_half_even(quo)
                assert qw[n, g * G + i] == max(-31, min(31, q))


@pytest.mark.parametrize("abits", [6, 8])
def test_quant_act_invariants(abits):
    qmax = 31 if abits == 6 else 127
    x = synth.activations(synth.derive_seed(5, abits), 16, 8 * G)
    qa, sa = oracle.quant_act(x, abits)
    xf = x.astype(np.float64).reshape(16, 8, G)
    q = qa.astype(np.float64).reshape(16, 8, G)
    s = sa.astype(np.float64)[:, :, None]
    assert np.abs(qa).max() <= qmax
    # |x - q*s| <= s/2, evaluated exactly in binary64 (products of a small int and a
    # binary32 are exact there); the slack covers a quotient rounded onto a tie.
    err = np.abs(xf - q * s)
    assert np.all(err <= s * (0.5 + 2.0 ** -18))
    # the largest magnitude in a group maps to +-qmax
    idx = np.argmax(np.abs(xf), axis=2)
    top = np.take_along_axis(q, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == qmax)
    # odd symmetry and power-of-two equivariance
    qn, sn = oracle.quant_act(-x, abits)
    assert np.array_equal(qn, -qa) and np.array_equal(sn, sa)
    q2, s2 = oracle.quant_act((x.astype(np.float32) * 2).astype(np.float16), abits)
    assert np.array_equal(q2, qa) and np.array_equal(s2, 2 * sa)


def test_quant_w6_invariants():
    w = synth.weights(synth.derive_seed(6), 32, 8 * G)
    qw, sw = oracle.quant_w6(w)
    wf = w.astype(np.float64).reshape(32, 8, G)
    q = qw.astype(np.float64).reshape(32, 8, G)
    s = sw.astype(np.float64)[:, :, None]
    assert np.abs(qw).max() <= 31
    assert np.all(np.abs(wf - q * s) <= s * (0.5 + 2.0 ** -18))
    idx = np.argmax(np.abs(wf), axis=2)
    top = np.take_along_axis(q, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == 31)
    qn, sn = oracle.quant_w6(-w)
    assert np.array_equal(qn, -qw) and np.array_equal(sn, sw)
    q2, s2 = oracle.quant_w6((w.astype(np.float32) * 2).astype(np.float16))
    assert np.array_equal(q2, qw)
    assert np.array_equal(s2.astype(np.float32), 2 * sw.astype(np.float32))


def test_quant_zero_groups():
    x = np.zeros((2, 2 * G), np.float16)
    x[1, G + 3] = -0.25
    qa, sa = oracle.quant_act(x, 6)
    assert sa[0, 0] == 0 and sa[0, 1] == 0 and sa[1, 0] == 0 and not qa[0].any()
    assert sa[1, 1] == np.float32(0.25) / np.float32(31) and qa[1, G + 3] == -31
    qw, sw = oracle.quant_w6(np.zeros((16, 2 * G), np.float16))
    assert not qw.any() and not sw.view(np.uint16).any()


def test_quant_w6_scale_underflow_gives_zero_codes():
    # amax / 31 rounds to +0 in fp16 (below half the smallest subnormal): codes are 0
    w = np.zeros((16, G), np.float16)
    w[0, 0] = np.float16(2.0 ** -24)  # smallest fp16 subnormal
    qw, sw = oracle.quant_w6(w)
    assert sw[0, 0].view(np.uint16) == 0 and not qw[0].any()


def test_quant_act_ramp_worked_example():
    """x[k] = (k-64)/64: amax = 1, s = fp32(1/31), and each code equals the
    half-to-even rounding of the exact rational quotient, except at x = +-0.5
    where the exact quotient is within one binary32 ulp of the tie 15.5 and the
    IEEE binary32 quotient (numpy) decides."""
    x = ((np.arange(G) - 64) / 64.0).astype(np.float16)[None, :]
    qa, sa = oracle.quant_act(x, 6)
    s = np.float32(1.0) / np.float32(31.0)
    assert sa[0, 0] == s and sa[0, 0].view(np.uint32) == 0x3D042108
    for k in range(G):
        quo = Fraction(k - 64, 64) / Fraction(float(s))
        if k in (32, 96):
            assert _near_tie(quo)
            assert qa[0, k] == int(np.rint(np.float32((k - 64) / 64) / s))
        else:
            assert not _near_tie(quo)
            assert qa[0, k] == round(quo)
    assert list(qa[0, :4]) == [-31, -31, -30, -30] and qa[0, 127] == 31


# ---------------------------------------------------------------------------
# integer group dots and the fused-dequantization accumulation
# ---------------------------------------------------------------------------

def _dequant(q, s, group=G):
    return q.astype(np.float64) * np.repeat(s.astype(np.float64), group, axis=1)


@pytest.mark.parametrize("abits", [6, 8])
def test_group_dots_match_numpy_integer_matmul(abits):
    qmax = 31 if abits == 6 else 127
    rng = np.random.default_rng(abits)
    M, N, K = 5, 48, 6 * G
    qa = rng.integers(-qmax, qmax + 1, (M, K)).astype(np.int8)
    qw = rng.integers(-31, 32, (N, K)).astype(np.int8)
    d = oracle.group_dots(qa, qw, nthreads=3)
    for g in range(K // G):
        ref = qa[:, g * G:(g + 1) * G].astype(np.int64) @ qw[:, g * G:(g + 1) * G].astype(np.int64).T
        assert np.array_equal(d[:, :, g], ref)
    # extreme operands reach the documented bound exactly
    qa[:] = qmax
    qw[:] = -31
    d = oracle.group_dots(qa, qw)
    assert np.all(d == -31 * qmax * G)


def test_group_dots_permutation_invariant_within_group():
    rng = np.random.default_rng(9)
    qa = rng.integers(-31, 32, (3, 2 * G)).astype(np.int8)
    qw = rng.integers(-31, 32, (16, 2 * G)).astype(np.int8)
    perm = np.concatenate([rng.permutation(G), G + rng.permutation(G)])
    assert np.array_equal(oracle.group_dots(qa, qw), oracle.group_dots(qa[:, perm], qw[:, perm]))


def _prepared(seed, M, N, K, abits):
    x = synth.activations(synth.derive_seed(seed, "x"), M, K)
    w = synth.weights(synth.derive_seed(seed, "w"), N, K)
    qa, sa = oracle.quant_act(x, abits)
    qw, sw = oracle.quant_w6(w)
    return qa, sa, qw, sw


@pytest.mark.parametrize("abits", [6, 8])
def test_gemm_within_fp32_bound_of_fp64_brute_force(abits):
    M, N, K = 7, 32, 5 * G
    qa, sa, qw, sw = _prepared(21 + abits, M, N, K, abits)
    y, acc, S = oracle.gemm(qa, sa, qw, sw, want_acc=True)
    y64 = _dequant(qa, sa) @ _dequant(qw, sw).T          # textbook dense matmul, binary64
    Gn = K // G
    bound = (Gn + 2) * 2.0 ** -24 * S + 1e-300
    assert np.all(np.abs(acc.astype(np.float64) - y64) <= bound)
    assert np.array_equal(y.view(np.uint16), acc.astype(np.float16).view(np.uint16))


def test_gemm_power_of_two_scales_are_exact():
    """s_w = 2^-10, s_a = 1: every step is exact, so Y is the integer matmul times 2^-10."""
    rng = np.random.default_rng(4)
    M, N, K = 4, 16, 3 * G
    qa = rng.integers(-31, 32, (M, K)).astype(np.int8)
    qw = rng.integers(-31, 32, (N, K)).astype(np.int8)
    sa = np.ones((M, K // G), np.float32)
    sw = np.full((N, K // G), 2.0 ** -10, np.float16)
    y, acc, _ = oracle.gemm(qa, sa, qw, sw, want_acc=True)
    exact = (qa.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64) * 2.0 ** -10
    assert np.array_equal(acc.astype(np.float64), exact)
    assert np.array_equal(y.view(np.uint16), exact.astype(np.float16).view(np.uint16))


def test_gemm_scaling_activation_scales_by_two_doubles_output():
    qa, sa, qw, sw = _prepared(31, 3, 16, 4 * G, 6)
    y1, a1, _ = oracle.gemm(qa, sa, qw, sw, want_acc=True)
    y2, a2, _ = oracle.gemm(qa, sa * np.float32(2), qw, sw, want_acc=True)
    assert np.array_equal(a2, 2 * a1)
    assert np.array_equal(y2.astype(np.float32), 2 * y1.astype(np.float32))


def _fp32_round(fr: Fraction) -> np.float32:
    """Correctly rounded (half to even) binary32 value of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    lo = np.float32(float(fr))
    # step to the neighbours that bracket fr
    while Fraction(float(lo)) > fr:
        lo = np.nextafter(lo, np.float32(-np.inf))
    while Fraction(float(np.nextafter(lo, np.float32(np.inf)))) <= fr:
        lo = np.nextafter(lo, np.float32(np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl, dh = fr - Fraction(float(lo)), Fraction(float(hi)) - fr
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (int(np.float32(lo).view(np.uint32)) & 1) == 0 else hi


def test_gemm_accumulation_in_exact_rationals():
    """Replays t = RN32(d*s_w), acc = RN32(t*s_a + acc) in exact rationals with an
    explicit binary32 rounding; the oracle must agree bit for bit."""
    qa, sa, qw, sw = _prepared(41, 2, 16, 6 * G, 8)
    y, acc, _ = oracle.gemm(qa, sa, qw, sw, want_acc=True)
    for m in range(2):
        for n in range(16):
            a = np.float32(0.0)
            for g in range(6):
                d = int(np.dot(qa[m, g * G:(g + 1) * G].astype(np.int64),
                               qw[n, g * G:(g + 1) * G].astype(np.int64)))
                t = _fp32_round(Fraction(d) * Fraction(float(sw[n, g])))
                a = _fp32_round(Fraction(float(t)) * Fraction(float(sa[m, g])) + Fraction(float(a)))
            assert a.view(np.uint32) == acc[m, n].view(np.uint32)


def test_gemm_packed_equals_gemm_on_codes_and_pack_w6_equals_quant_then_pack():
    x = synth.activations(synth.derive_seed(51, "x"), 3, 3 * G)
    w = synth.weights(synth.derive_seed(51, "w"), 32, 3 * G)
    qa, sa = oracle.quant_act(x, 6)
    qw, sw = oracle.quant_w6(w)
    wp, sw2 = oracle.pack_w6(w)
    assert np.array_equal(sw.view(np.uint16), sw2.view(np.uint16))
    assert np.array_equal(wp, oracle.pack_codes(qw))
    assert np.array_equal(oracle.gemm(qa, sa, qw, sw).view(np.uint16),
                          oracle.gemm_packed(qa, sa, wp, sw, 32).view(np.uint16))


def test_gemm_threading_does_not_change_results():
    qa, sa, qw, sw = _prepared(61, 4, 64, 2 * G, 6)
    y1 = oracle.gemm(qa, sa, qw, sw, nthreads=1)
    y7 = oracle.gemm(qa, sa, qw, sw, nthreads=7)
    assert np.array_equal(y1.view(np.uint16), y7.view(np.uint16))


def test_quantized_layer_tracks_fp64_reference():
    """Sanity only (the pages report accuracy as perplexity, so this is not a pin):
    the W6A8 / W6A6 layer stays close to the unquantized fp64 product."""
    x = synth.activations(synth.derive_seed(71, "x"), 8, 8 * G)
    w = synth.weights(synth.derive_seed(71, "w"), 64, 8 * G)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    for abits, limit in [(8, 3e-3), (6, 2e-2)]:
        qa, sa = oracle.quant_act(x, abits)
        qw, sw = oracle.quant_w6(w)
        y = oracle.gemm(qa, sa, qw, sw).astype(np.float64)
        nmse = np.sum((y - ref) ** 2) / np.sum(ref ** 2)
        assert nmse < limit, (abits, nmse)


# ---------------------------------------------------------------------------
# worked vectors (tests/golden/worked_vectors.txt), re-derived here in exact
# rational arithmetic before the oracle is compared with them
# ---------------------------------------------------------------------------

def _golden_vectors():
    ramp, e2e = None, {}
    with open(os.path.join(GOLDEN, "worked_vectors.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split(";")]
            if parts[0] == "w6_ramp":
                ramp = (int(parts[1].split()[1], 16), [int(v) for v in parts[2].split()[1:]],
                        [int(v) for v in parts[3].split()[1:]])
            elif parts[0] == "e2e":
                e2e[int(parts[1])] = dict(
                    d=[int(v) for v in parts[2].split()],
                    sa=[int(v, 16) for v in parts[3].split()],
                    sw=[int(v, 16) for v in parts[4].split()],
                    acc=int(parts[5], 16), y=int(parts[6], 16))
    return ramp, e2e


def _exact_codes(vals, scale, qmax):
    """round_half_even(v / scale) in exact rationals, clamped; a quotient within
    2^-18 of a rounding boundary is left to the IEEE binary32 quotient (numpy)."""
    out = []
    for v in vals:
        quo = Fraction(float(v)) / Fraction(float(scale))
        q = int(np.rint(np.float32(v) / np.float32(scale))) if _near_tie(quo) else round(quo)
        out.append(max(-qmax, min(qmax, q)))
    return out


def _worked_inputs():
    k = np.arange(G)
    x = np.zeros((1, 2 * G), np.float16)
    w = np.zeros((16, 2 * G), np.float16)
    x[0, :G] = (k - 64) / 64.0
    w[0, :G] = 0.05 * (k - 64) / 64.0
    x[0, G:] = -3.0 * (63 - k) / 64.0
    w[0, G:] = 0.02 * np.sin(k.astype(np.float64))
    return x, w


def test_w6_ramp_worked_vector():
    s16_bits, head, tail = _golden_vectors()[0]
    k = np.arange(G)
    w = np.zeros((16, G), np.float16)
    w[0] = 0.05 * (k - 64) / 64.0
    # independent derivation: IEEE division (numpy), fp16 rounding, exact rational codes
    amax = np.max(np.abs(w[0].astype(np.float32)))
    s16 = (np.float32(amax) / np.float32(31)).astype(np.float16)
    assert int(s16.view(np.uint16)) == s16_bits
    codes = _exact_codes(w[0], s16, 31)
    assert codes[:4] == head and codes[124:] == tail
    qw, sw = oracle.quant_w6(w)
    assert int(sw[0, 0].view(np.uint16)) == s16_bits
    assert list(qw[0]) == codes


@pytest.mark.parametrize("abits", [6, 8])
def test_end_to_end_worked_vector(abits):
    ref = _golden_vectors()[1][abits]
    qmax = 31 if abits == 6 else 127
    x, w = _worked_inputs()
    # independent derivation of every intermediate
    acc = np.float32(0.0)
    for g in range(2):
        xs, ws = x[0, g * G:(g + 1) * G], w[0, g * G:(g + 1) * G]
        s_a = np.float32(np.max(np.abs(xs.astype(np.float32)))) / np.float32(qmax)
        s16 = (np.float32(np.max(np.abs(ws.astype(np.float32)))) / np.float32(31)).astype(np.float16)
        qa = _exact_codes(xs, s_a, qmax)
        qw = _exact_codes(ws, s16, 31)
        d = sum(a * b for a, b in zip(qa, qw))
        assert d == ref["d"][g]
        assert int(s_a.view(np.uint32)) == ref["sa"][g]
        assert int(s16.view(np.uint16)) == ref["sw"][g]
        t = _fp32_round(Fraction(d) * Fraction(float(s16)))
        acc = _fp32_round(Fraction(float(t)) * Fraction(float(s_a)) + Fraction(float(acc)))
    assert int(acc.view(np.uint32)) == ref["acc"]
    assert int(np.float32(acc).astype(np.float16).view(np.uint16)) == ref["y"]
    # the oracle, step by step
    qa, sa = oracle.quant_act(x, abits)
    qw, sw = oracle.quant_w6(w)
    assert [int(v) for v in sa[0].view(np.uint32)] == ref["sa"]
    assert [int(v) for v in sw[0].view(np.uint16)] == ref["sw"]
    assert list(oracle.group_dots(qa, qw[:1])[0, 0]) == ref["d"]
    y, acc_o, _ = oracle.gemm(qa, sa, qw[:1], sw[:1], want_acc=True)
    assert int(acc_o[0, 0].view(np.uint32)) == ref["acc"]
    assert int(y[0, 0].view(np.uint16)) == ref["y"]
    # the same through the packed weights
    wp, sw2 = oracle.pack_w6(w)
    assert int(oracle.gemm_packed(qa, sa, wp, sw2, 16)[0, 0].view(np.uint16)) == ref["y"]


# ---------------------------------------------------------------------------
# the oracle's C code under the address and undefined-behaviour sanitizers
# ---------------------------------------------------------------------------

def test_oracle_runs_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """tests/oracle_sanitize_driver.c runs every oracle function (ordinary, zero,
    extreme and subnormal groups; 1 and several threads; argument errors) in a gcc
    build of oracle/flexq_oracle.c with -fsanitize=address,undefined; any memory or
    undefined-behaviour error aborts the run."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    here = os.path.dirname(os.path.abspath(__file__))
    exe = str(tmp_path / "oracle_sanitized")
    subprocess.check_call([gcc, "-std=c11", "-O1", "-g", "-pthread", "-ffp-contract=off",
                           "-fno-fast-math", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           os.path.join(here, "oracle_sanitize_driver.c"),
                           os.path.join(os.path.dirname(here), "oracle", "flexq_oracle.c"),
                           "-o", exe, "-lm"])
    # (verify_asan_link_order=0: the environment may preload a library ahead of ASan's)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout
