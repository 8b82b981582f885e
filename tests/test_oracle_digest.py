"""The oracle's tiny-workload outputs still hash to the committed digest (drift guard)."""

import json
import os

import golden.make_tiny_digest as mk


def test_tiny_digest_unchanged():
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "tiny_oracle_digest.json")) as f:
        want = json.load(f)
    assert mk.digests() == want
