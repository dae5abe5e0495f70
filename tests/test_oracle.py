"""The oracle against its pins (CPU only)."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_golden_snapshot():
    """The oracle still reproduces the snapshot written from it by
    tests/golden/make_golden.py (regression guard, not a pin)."""
    import json
    import os

    import numpy as np

    import oracle
    from prefill_decode_amd import inputs

    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_snapshot.json")
    doc = json.load(open(path))
    s = dict(doc["spec"])
    spec = inputs.custom_spec(s.pop("name"), s.pop("num_qo_heads"), s.pop("num_kv_heads"),
                              [tuple(p) for p in s.pop("prefill")], s.pop("decode_kv"), **s)
    out = oracle.batch_attention(inputs.make_batch_host(spec), workers=1)
    for k, shape in doc["shapes"].items():
        want = np.array([float.fromhex(x) for x in doc[k]]).reshape(shape)
        assert np.max(np.abs(out[k] - want)) <= 1e-13, k
