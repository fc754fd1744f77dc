"""The oracle still reproduces the committed tiny-workload fixture."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_tiny_oracle_fixture_unchanged():
    want = json.load(open(os.path.join(HERE, "golden", "tiny_oracle.json")))
    want.pop("_about")
    got = json.loads(json.dumps(make_golden.compute(), sort_keys=True))
    assert got == want
