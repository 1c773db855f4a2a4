"""The CPU oracle against what the pages and plain mathematics fix (no GPU)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    ok, detail = pin(oracle.scan)
    assert ok, detail


def test_golden_bits_reproduce_printed_parity():
    """The fixture's bit recipe reproduces the parity the page prints."""
    g, bits = pins._parity_bits()
    assert int(bits.sum() % 2) == g["parity"]
    n = g["decay_steps"]
    direct = 1.0
    for bit in bits[:n]:
        direct *= g["decay_factor_bit1"] if bit else g["decay_factor_bit0"]
    assert round(direct, 6) == g["decay_final_rounded_6dp"]


def test_oracle_rejects_bad_shapes():
    import numpy as np
    z = np.zeros
    # H = 3 heads cannot be split into G = 2 groups
    with pytest.raises(ValueError):
        oracle.scan(z((1, 3, 3, 1, 2)), z((1, 3, 3)), z(3), z((1, 3, 3)), z((1, 3, 2, 2)),
                    z((1, 3, 2, 1, 4)), z((1, 3, 2, 1, 4)), z(3))
    # odd state size N = 3
    with pytest.raises(ValueError):
        oracle.scan(z((1, 3, 2, 1, 2)), z((1, 3, 2)), z(2), z((1, 3, 2)), z((1, 3, 1, 1)),
                    z((1, 3, 1, 1, 3)), z((1, 3, 1, 1, 3)), z(2))


def test_oracle_empty_sequence():
    """L = 0: no outputs, state_out = state_in."""
    import numpy as np
    d = pins.rand_case(b=1, L=4, H=2, G=1, P=3, N=4, R=2)
    d0 = {k: (v[:, :0] if v.ndim > 1 else v) for k, v in d.items()}
    st = pins.rand_state(d)
    y, h = oracle.scan(*pins._args(d0), state_in=st)
    assert y.shape[1] == 0
    assert np.array_equal(h, st[0])
