"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle)


def test_zero_padding_embeds_layer_exactly():
    """The zero-padding used to run tiny fixtures on the GPU leaves the
    oracle's routing and output unchanged."""
    import numpy as np
    from common import layer_from_json
    from gpu_helpers import padded_layer
    for f in ("worked_example_routed.json", "worked_example_shared.json"):
        j, layer, x = layer_from_json(f)
        big = padded_layer(layer, 64, 64, 64)
        xp = np.zeros((x.shape[0], 64), np.float32)
        xp[:, :2] = x
        rt0, y0 = oracle.forward(layer, x)
        rt1, y1 = oracle.forward(big, xp)
        assert np.array_equal(rt0.idx, rt1.idx) and np.array_equal(rt0.mask_bits, rt1.mask_bits)
        assert np.array_equal(y1[:, :2], y0) and np.all(y1[:, 2:] == 0)
