"""CPU pins of the oracle (no GPU needed)."""

import pytest

import oracle.csa_oracle as O
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_near_decision_mask_on_seeded_latents():
    """The seeded N(0,1) latents put no pooled element within 1e-12 of a
    rounding decision, so bit-exact parity of cache bytes is well posed."""
    import numpy as np
    rng = np.random.default_rng(0)
    kv = rng.standard_normal((4096, 128)).astype(np.float32)
    g = rng.standard_normal(4096).astype(np.float32)
    assert not O.near_decision_mask(kv, g, 4).any()
    # and the mask does fire on a value placed on a midpoint
    kv2 = np.zeros((4, 32), np.float32)
    kv2[:, 0] = 4.0
    kv2[:, 1] = 1.25
    assert O.near_decision_mask(kv2, np.zeros(4, np.float32), 4)[0, 1]
