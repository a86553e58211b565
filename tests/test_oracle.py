"""The fp64 oracle against its pins (CPU only), plus argument handling."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.gdn_forward)


@pytest.mark.parametrize("pin", oracle_pins.CONV_PINS, ids=lambda p: p.__name__)
def test_oracle_short_conv_pin(pin):
    pin(oracle.short_conv)


@pytest.mark.parametrize("pin", oracle_pins.GRAD_PINS, ids=lambda p: p.__name__)
def test_oracle_gradient_pin(pin):
    pin(oracle.gdn_backward, oracle.gdn_forward)


@pytest.mark.parametrize("pin", oracle_pins.PRE_PINS, ids=lambda p: p.__name__)
def test_oracle_preprocessing_pin(pin):
    pin(oracle.preprocess, oracle.gdn_forward)


@pytest.mark.parametrize("pin", oracle_pins.PRE_GRAD_PINS, ids=lambda p: p.__name__)
def test_oracle_preprocessing_gradient_pin(pin):
    pin(oracle.preprocess_backward, oracle.preprocess)


@pytest.mark.parametrize("pin", oracle_pins.CONV_GRAD_PINS, ids=lambda p: p.__name__)
def test_oracle_short_conv_gradient_pin(pin):
    pin(oracle.short_conv_backward, oracle.short_conv)


def test_oracle_fused_layer_gradient_chain():
    oracle_pins.pin_fused_layer_chain(oracle.preprocess_backward, oracle.preprocess, oracle.gdn_backward,
                                      oracle.gdn_forward)


def test_bruteforce_is_not_the_recurrence():
    """The brute force must itself respect the transition-product algebra: with
    one token and S0 = 0 it reduces to beta v k^T, whatever the gate."""
    c = oracle_pins.random_case(5, [1], hk=1, hv=1, dk=3, dv=2, with_h0=False)
    _, hT = oracle_pins.bruteforce(c)
    expect = float(c["beta"][0, 0]) * np.outer(c["v"][0, 0].astype(np.float64), c["k"][0, 0].astype(np.float64))
    np.testing.assert_allclose(hT[0, 0], expect, rtol=1e-12)


def test_zero_sequences_is_a_noop():
    c = oracle_pins.random_case(1, [], hk=1, hv=1, dk=2, dv=2, with_h0=False)
    out, hT = oracle.gdn_forward(**c)
    assert out.shape == (0, 1, 2) and hT.shape == (0, 1, 2, 2)


def test_rejects_bad_grouping():
    c = oracle_pins.random_case(2, [3], hk=2, hv=3, dk=2, dv=2)
    with pytest.raises(ValueError):
        oracle.gdn_forward(**c)


def test_rejects_mixed_io_dtypes():
    import torch
    c = oracle_pins.random_case(3, [3], hk=1, hv=1, dk=2, dv=2)
    c["q"] = torch.from_numpy(c["q"]).to(torch.bfloat16)
    with pytest.raises(TypeError):
        oracle.gdn_forward(**c)


def test_thread_count_does_not_change_bits():
    c = oracle_pins.random_case(4, [5, 7, 2], hk=2, hv=4, dk=8, dv=8)
    o1, s1 = oracle.gdn_forward(**c, n_threads=1)
    o4, s4 = oracle.gdn_forward(**c, n_threads=4)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)
