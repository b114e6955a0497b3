"""The seeded input generator: reproducibility, bf16 rounding, shapes."""

import numpy as np

from synth import Inputs, WORKLOADS, bf16_bits, bf16_round, get_workload, sample_tokens


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4,
                     -2.5, 3.0e-39, 65504.0], dtype=np.float32)
    bits = bf16_bits(vals)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80        # tie -> even mantissa
    assert bits[2] == 0x3F82        # tie -> even mantissa (rounds up)
    assert bits[3] == 0x3F80
    assert bits[4] == 0xC020
    r = bf16_round(vals)
    np.testing.assert_array_equal(bf16_round(r), r)  # idempotent
    normal = np.abs(vals) > 1e-37  # relative bound holds for normal numbers
    assert np.all(np.abs(r - vals)[normal] <= np.abs(vals)[normal] * 2.0 ** -8)


def test_draws_are_reproducible_and_independent_of_order():
    w = WORKLOADS["tiny"]
    a, b = Inputs(w), Inputs(w)
    q_late = b.query(3)
    np.testing.assert_array_equal(a.row(2), b.row(2))
    np.testing.assert_array_equal(a.query(3), q_late)
    np.testing.assert_array_equal(a.dout(4), b.dout(4))
    assert not np.array_equal(a.row(0), a.row(1))


def test_shapes_and_distributions():
    w = get_workload("mhar1b@T64")
    x = Inputs(w)
    assert w.tokens == 64 and w.sites == 73 and w.rows == 73
    row = x.row(5)
    assert row.shape == (64, 1280) and row.dtype == np.float32
    np.testing.assert_array_equal(bf16_round(row), row)  # exactly bf16 values
    assert 0.5 <= x.scales[5] <= 2.0
    q = x.query(0)
    assert q.shape == (1280,) and 0.01 < q.std() < 0.03
    lr = Inputs(get_workload("lr_h8@T16"))
    assert lr.extra(0).shape == (16, 7168)
    assert lr.query(0).shape == (1792,)
    np.testing.assert_array_equal(lr.scales, 1.0)


def test_sample_tokens():
    s = sample_tokens(1000, 50)
    assert s[0] == 0 and s[-1] == 999 and len(np.unique(s)) == len(s)
    assert np.all(np.diff(s) > 0)
