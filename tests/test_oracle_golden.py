"""Regression guard: the oracle's output for the tiny workload is frozen in
tests/golden/tiny_oracle.json (written by tests/golden/make_golden.py, which
calls only the oracle).  Any change of the oracle's arithmetic must come with a
regenerated fixture and a commit message naming the passage that justifies it."""
import json
import os

from tests.golden.make_golden import digests

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_digests_unchanged(oracle_lib):
    want = json.load(open(os.path.join(HERE, "golden", "tiny_oracle.json")))
    assert digests() == want
