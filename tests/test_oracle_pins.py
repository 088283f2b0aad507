"""CPU pins of the oracle (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_golden_regression():
    """The oracle still reproduces the fixture written by tests/golden/make_golden.py."""
    import json
    import os

    import numpy as np

    import oracle
    from swa_inputs import PrefillConfig, prefill_inputs

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_tiny.json")
    data = json.load(open(path))
    for name, entry in data.items():
        cfg = PrefillConfig(**entry["config"])
        q, k, v, sinks = prefill_inputs(cfg)
        o = oracle.prefill(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale)
        assert np.abs(o - np.array(entry["o"])).max() < 1e-13, name
