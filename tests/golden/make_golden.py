"""Writes tests/golden/oracle_snapshot.json from the oracle alone.

The pages print no worked example with numbers (no inputs/outputs of an
attention call appear in them), so this folder holds no page values.  The
snapshot here is written only by this script, which calls only ``oracle/``
(and the seeded input generator): it freezes the pinned oracle's output on a
small batch so that a later, unnoticed change to the oracle's arithmetic
shows up as a failing test.  Re-run it only together with a change to the
oracle whose justification (the passage or reading) is stated.

    python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from prefill_decode_amd import inputs  # noqa: E402

SPEC = dict(name="golden", num_qo_heads=4, num_kv_heads=2,
            prefill=[(3, 10), (2, 2)], decode_kv=[5, 1], seed=4242,
            head_dim=8, page_size=4, extra_pages=2)


def main():
    s = dict(SPEC)
    spec = inputs.custom_spec(s.pop("name"), s.pop("num_qo_heads"),
                              s.pop("num_kv_heads"), s.pop("prefill"),
                              s.pop("decode_kv"), **s)
    b = inputs.make_batch_host(spec)
    out = oracle.batch_attention(b, workers=1)
    doc = {"spec": SPEC,
           "note": "written by tests/golden/make_golden.py from oracle/ only",
           **{k: [float.hex(float(x)) for x in v.ravel()] for k, v in out.items()},
           "shapes": {k: list(v.shape) for k, v in out.items()}}
    with open(os.path.join(os.path.dirname(__file__), "oracle_snapshot.json"), "w") as f:
        json.dump(doc, f, indent=0)


if __name__ == "__main__":
    main()
