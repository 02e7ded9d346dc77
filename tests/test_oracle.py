"""The CPU oracle against what the pages and the mathematics fix (not gpu)."""
import numpy as np
import pytest

import oracle
import synth

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def test_within_bound_zero_scale():
    y_ref = np.zeros((1, 2))
    a = np.zeros((1, 2))
    assert within_all(np.array([[0.0, -0.0]]), y_ref, a)
    assert not within_all(np.array([[1e-30, 0.0]]), y_ref, a)


def within_all(y, r, a):
    return bool(np.all(oracle.within_bound(y, r, a)))


def test_i64_rejects_non_integers():
    x = synth.f32_to_bf16_bits(np.array([[0.5, 1.0]], np.float32))
    w = synth.f32_to_bf16_bits(np.array([[1.0, 1.0]], np.float32))
    with pytest.raises(ValueError):
        oracle.gemm_i64(x, w)


def test_grouped_rejects_bad_offsets():
    x = synth.normal_bf16(1, (4, 8))
    w = synth.normal_bf16(2, (2, 3, 8))
    for off in ([0, 3, 2], [1, 2, 4], [0, 2, 5]):
        with pytest.raises(ValueError):
            oracle.grouped_f64(x, w, np.array(off, np.int32))


def test_threads_do_not_change_values():
    x = synth.normal_bf16(3, (7, 512))
    w = synth.normal_bf16(4, (33, 512), 0.02)
    y1, a1 = oracle.gemm_f64(x, w, threads=1)
    y4, a4 = oracle.gemm_f64(x, w, threads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)
