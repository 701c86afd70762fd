"""Regression fixture: the oracle's tiny-workload outputs must not drift
silently.  Regenerate with tests/golden/make_golden.py (and say why in the
commit message) only when the oracle's arithmetic is deliberately changed."""
import json
import os

from tests.golden.make_golden import compute


def test_tiny_oracle_digests_unchanged():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    want = json.load(open(path))
    got = compute()
    for k, v in got.items():
        assert want[k] == v, k
