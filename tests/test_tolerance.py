"""Pins of the split-K tolerance check (tests/tolerance.py): fp16 ulps at known
values and the pass / fail decisions at the bounds."""
import numpy as np

import tolerance


def h(v):
    return np.array(v, np.float16).view(np.uint16)


def test_ulp16_values():
    vals = [1.0, 1.5, 0.75, 2.0, 65504.0, 2.0 ** -14, 2.0 ** -15, 0.0, -3.0, 1024.0]
    want = [2.0 ** -10, 2.0 ** -10, 2.0 ** -11, 2.0 ** -9, 32.0, 2.0 ** -24, 2.0 ** -24,
            2.0 ** -24, 2.0 ** -9, 1.0]
    assert np.array_equal(tolerance.ulp16(h(vals)), np.array(want))
    # the spacing really is the distance to the next fp16 number up
    for v in (1.0, 0.75, 3.0, 1000.0, 2.0 ** -20):
        nxt = np.nextafter(np.float16(v), np.float16(np.inf))
        assert float(nxt) - v == tolerance.ulp16(h([v]))[0]


def test_check_decisions():
    ref = h([1.0, 1.0, 1.0, 100.0])
    acc_ref = np.array([1.0, 1.0, 1.0, 100.0])
    S = np.array([10.0, 10.0, 10.0, 100.0])
    # one ulp off passes without looking at the accumulator
    ok, n_ulp, n_acc = tolerance.check(h([1.0 + 2 ** -10, 1.0, 1.0, 100.0]), ref,
                                       acc_ref + [1.0, 0, 0, 0], acc_ref, S)
    assert ok and n_ulp == 0 and n_acc == 1
    # two ulps off passes only with the fp32 sum inside 1e-5 * S
    y2 = h([1.0 + 2 ** -9, 1.0, 1.0, 100.0])
    assert tolerance.check(y2, ref, acc_ref + [9e-5, 0, 0, 0], acc_ref, S)[0]
    assert not tolerance.check(y2, ref, acc_ref + [1.1e-4, 0, 0, 0], acc_ref, S)[0]
    # exact agreement passes
    assert tolerance.check(ref, ref, acc_ref, acc_ref, S) == (True, 0, 0)


def test_check_overflowed_outputs():
    """An output that overflows fp16 agrees with the same infinity; a finite value or
    the other infinity is judged by the fp32 sums alone."""
    ref = h([np.inf, -np.inf, 1.0])
    acc_ref = np.array([7e4, -7e4, 1.0])
    S = np.array([7e4, 7e4, 1.0])
    with np.errstate(all="raise"):
        assert tolerance.check(ref, ref, acc_ref, acc_ref, S) == (True, 0, 0)
    # 65504 against +inf: more than an ulp apart, passes only on the fp32 sums
    y = h([65504.0, -np.inf, 1.0])
    assert tolerance.check(y, ref, acc_ref, acc_ref, S)[:2] == (True, 1)
    assert not tolerance.check(y, ref, acc_ref - [1.0, 0, 0], acc_ref, S)[0]
    assert not tolerance.check(h([-np.inf, -np.inf, 1.0]), ref, acc_ref - [2e4, 0, 0],
                               acc_ref, S)[0]
