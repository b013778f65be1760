"""The oracle still produces the outputs frozen in tests/golden (regression
guard; see tests/golden/README.md)."""
import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_frozen_digests():
    with open(os.path.join(HERE, "golden", "oracle_digests.json")) as f:
        frozen = json.load(f)
    now = make_golden.compute()
    assert set(now) == set(frozen)
    for name in frozen:
        assert now[name] == frozen[name], f"oracle output changed: {name}"
