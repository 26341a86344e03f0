"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_bwd_pins
import oracle_paged_pins
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_brute_force_full_grid(oracle_lib):
    """Every tiny shape of the grid: L in {1,2,3,7,17,64,130}, d in {64,128},
    (H,H_kv) in {(1,1),(4,2),(4,1)}, causal on/off, window in {-1,0,1,5}, fp16/bf16."""
    oracle_pins.pin_brute_force_full(oracle_lib)


def test_visible_count_brute():
    """The closed-form visible-key count used by the K = 0 pin, by enumeration."""
    for L in (1, 5, 33):
        for causal in (False, True):
            for window in (-1, 0, 1, 4, 40):
                for i in range(L):
                    n = 0
                    for j in range(L):
                        ok = (not causal or j <= i) and (
                            window < 0 or (i - j <= window and (causal or j - i <= window)))
                        n += ok
                    assert oracle_pins.visible_count(i, L, causal, window) == n


def test_oracle_rejects_bad_arguments(oracle_lib):
    import numpy as np
    import oracle
    q = np.zeros((1, 3, 4, 64), np.uint16)
    k = np.zeros((1, 2, 4, 64), np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, "f16", True, -1, 0.125, lib=oracle_lib)   # 3 % 2 != 0


@pytest.mark.parametrize("pin", oracle_paged_pins.ALL_PAGED_PINS, ids=lambda f: f.__name__)
def test_paged_pin(pin):
    from oracle import paged
    pin(paged)
