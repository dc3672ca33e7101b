"""The oracle still reproduces its stored tiny greedy run (regression anchor)."""
import json
import os

from tests.golden.make_golden import tiny_greedy


def test_tiny_greedy_run_unchanged():
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_greedy.json")) as f:
        want = json.load(f)
    got = tiny_greedy()
    assert got["prompt"] == want["prompt"]
    assert got["ids"] == want["ids"]
