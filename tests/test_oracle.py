"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_err_rms_metric():
    x = np.array([1.0, -1.0, 1.0, -1.0])
    assert oracle.err_rms(x + np.array([0, 0, 0.5, 0]), x) == 0.5
    assert oracle.err_rms(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.err_rms(np.array([0.0, 2e-3]), np.zeros(2)) == 2e-3
    assert oracle.err_rms(np.array([np.nan, 1.0]), np.ones(2)) == np.inf


def test_empty_sequence(orc):
    q = np.zeros((1, 0, 1, 4)); v = np.zeros((1, 0, 1, 3))
    a = np.zeros((1, 0, 1))
    s0 = np.arange(12.0).reshape(1, 1, 3, 4)
    o, sf = orc.gdn_fwd(q, q, v, a, a, s0)
    assert o.shape == (1, 0, 1, 3)
    np.testing.assert_array_equal(sf, s0)


def test_alpha_zero_resets(orc):
    """alpha = 0 forgets everything before the token: S_t = beta v k^T."""
    from oracle_pins import rand_gdn
    q, k, v, a, b, S0 = rand_gdn(30, T=4)
    a[:, 2] = 0.0
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    o2, sf2 = orc.gdn_fwd(q[:, 2:], k[:, 2:], v[:, 2:], a[:, 2:], b[:, 2:],
                          None)
    np.testing.assert_allclose(o[:, 2:], o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(sf, sf2, rtol=1e-14, atol=1e-15)
