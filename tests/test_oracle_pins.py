"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.FORWARD_PINS, ids=lambda p: p.__name__)
def test_forward_pin(lib, pin):
    pin(lib)


def test_fd_gradients(lib):
    pins.pin_fd_gradients(lib)


def test_l2norm_fd_gradients(lib):
    pins.pin_l2norm_fd(lib)
