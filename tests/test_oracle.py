"""The fp64 oracle against its pins (CPU only)."""
import pytest

from oracle import oracle as oracle_mod
from oracle.oracle import OracleError
from tests import oracle_pins
import torch


@pytest.fixture(scope="module")
def o():
    return oracle_mod.default()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_rejects_bad_arguments(o):
    codes = torch.full((4, 12), 8, dtype=torch.uint8)
    scales = torch.ones(3, 4, dtype=torch.float32)
    x = torch.ones(2, 12)
    with pytest.raises(OracleError):
        o.linear_fwd(x, codes, scales, 5)           # K % group_size != 0
    bad = codes.clone()
    bad[1, 3] = 16
    with pytest.raises(OracleError):
        o.linear_fwd(x, bad, scales, 4)             # code outside 0..15
    with pytest.raises(OracleError):
        o.linear_bwd_input(torch.ones(2, 5), codes, scales, 4)   # d_out not [M, N]


def test_threads_reported(o):
    assert o.threads_used(1) == 1
    assert o.threads_used(2) == 2
