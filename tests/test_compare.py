"""CPU: self-test of the comparison gates every parity test relies on.  A gate that cannot
fail proves nothing, so errors are planted on purpose (on the CPU, in copies of a reference
array) and each gate must catch and localise them:
* 1-ulp changes at three positions (interior, midpoint, last) fail the bitwise gate, which
  names all three;
* an error of twice the tolerance at one element fails the tolerance gate, which names it;
  half the tolerance everywhere passes."""
import numpy as np
import pytest

from compare import assert_bitwise, assert_within, report, tolerance


def _ref(n=1001, dtype=np.float32):
    return np.random.default_rng(20260908).standard_normal(n).astype(dtype)


def test_bitwise_gate_catches_and_localises_one_ulp():
    ref = _ref()
    got = ref.copy()
    planted = [123, ref.size // 2, ref.size - 1]
    for i in planted:
        got[i] = np.nextafter(got[i], np.float32(np.inf))
    with pytest.raises(AssertionError) as e:
        assert_bitwise(got, ref, "planted")
    msg = str(e.value)
    assert "3 of 1001 elements differ" in msg
    for i in planted:
        assert f"({i},)" in msg, (i, msg)
    assert_bitwise(ref.copy(), ref, "identical copy")


def test_bitwise_gate_on_16_bit_patterns():
    ref = _ref().astype(np.float16).view(np.uint16)
    got = ref.copy()
    got[7] ^= 1
    with pytest.raises(AssertionError):
        assert_bitwise(got, ref, "f16 pattern")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tolerance_gate_catches_twice_the_bar(dtype):
    atol, rtol = tolerance(dtype)
    ref = _ref().astype(np.float64)
    bar = atol + rtol * np.abs(ref)
    assert_within(ref + 0.5 * bar, ref, atol, rtol, "half the bar")
    got = ref.copy()
    got[ref.size // 2] += 2.0 * bar[ref.size // 2]
    with pytest.raises(AssertionError) as e:
        assert_within(got, ref, atol, rtol, "twice the bar")
    assert f"({ref.size // 2},)" in str(e.value)


def test_tolerance_gate_treats_nan_as_a_failure_unless_both_nan():
    ref = _ref().astype(np.float64)
    got = ref.copy()
    got[5] = np.nan
    with pytest.raises(AssertionError):
        assert_within(got, ref, 1e-5, 0.0, "NaN in the result only")
    ref2 = ref.copy()
    ref2[5] = np.nan
    assert_within(got, ref2, 1e-5, 0.0, "NaN on both sides (a poisoned byte)")


def test_report_fields():
    ref = _ref()
    got = ref.copy()
    got[3] += np.float32(1e-3)
    r = report(got, ref, 1e-5, 0.0)
    assert r.n == ref.size and r.worst == (3,) and r.failing == [(3,)]
    assert abs(r.max_abs - abs(float(got[3]) - float(ref[3]))) < 1e-12
    assert abs(r.bitwise_pct - 100.0 * (ref.size - 1) / ref.size) < 1e-9
